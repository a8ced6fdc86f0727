"""Replay a synthetic trace through the oracle (tests and CPU baseline only).

Order of one decode step t for one layer group, as the engine runs it: the
step's appended positions first (so they can be selected at once), then the
group's step over all of its selection sets, then one gather per layer of the
group (the layers share one selection, UlaCache summary section 2).
"""

from __future__ import annotations

from typing import Iterator, Optional

import numpy as np

from synth import rows_for
from .pblru import PBLRUGroup

LOAD_CHUNK = 1 << 18


def new_group(trace, full_data: bool = True, placement: str = "lowest") -> PBLRUGroup:
    wl = trace.wl
    return PBLRUGroup(trace.N, trace.P, trace.H, wl.ring, wl.layers, wl.row_bytes, full_data,
                      placement=placement)


def initial_load(grp: PBLRUGroup, trace, g: int) -> None:
    wl = trace.wl
    order = trace.initial_load_order()
    for s in range(0, order.size, LOAD_CHUNK):
        las = order[s:s + LOAD_CHUNK]
        rows = rows_for(wl.seed, g, las, wl.layers, wl.row_bytes) if grp.full_data else None
        grp.append(las, rows)


def replay(trace, g: int, full_data: bool = True, gather: bool = True,
           steps: Optional[int] = None, selections=None) -> Iterator[tuple]:
    """Yield (t, sel, group, gathered) after every step; gathered is a list per layer."""
    wl = trace.wl
    grp = new_group(trace, full_data)
    initial_load(grp, trace, g)
    sels = trace.selections(g) if selections is None else iter(selections)
    last = trace.steps if steps is None else steps
    for t in range(1, last + 1):
        sel = next(sels)
        app = trace.appends(t)
        grp.append(app, rows_for(wl.seed, g, app, wl.layers, wl.row_bytes) if full_data else None)
        grp.step(sel)
        outs = [grp.gather(sel, l, step=t) for l in range(wl.layers)] if (gather and full_data) else None
        yield t, sel, grp, outs
