"""Drive a decode trace through the engine (initial load, then per step: appends,
the group's step, one gather per layer). Used by the GPU tests and bench.py.

The trace object supplies the addresses (initial_load_order, appends(t),
selections(g)); `rows(las, g)` supplies the appended rows as a CUDA tensor.
"""

from __future__ import annotations

import numpy as np

from .ula import Engine

LOAD_CHUNK = 1 << 18


def engine_for(trace, max_append: int = 1 << 16, policy: int = 0) -> Engine:
    wl = trace.wl
    return Engine(num_groups=wl.groups, layers=wl.layers, row_bytes=wl.row_bytes, ring=wl.ring,
                  logical_capacity=trace.N, gpu_slots=trace.P, host_slots=trace.H,
                  max_sets=trace.n_sets, max_k=trace.k, max_append=max_append, policy=policy)


def initial_load(eng: Engine, trace, groups, rows) -> None:
    order = trace.initial_load_order()
    for g in groups:
        for s in range(0, order.size, LOAD_CHUNK):
            las = order[s:s + LOAD_CHUNK]
            eng.append(g, las, rows(las, g))


def step_all(eng: Engine, trace, t: int, sels, groups, rows, outs=None):
    """Step t for the given groups. sels[g]: CUDA int32 [n_sets][k]. Returns gathered tensors."""
    app = trace.appends(t)
    gathered = {}
    for g in groups:
        if app.size:
            eng.append(g, app, rows(app, g))
        eng.step(g, sels[g])
        gathered[g] = [eng.gather(g, l, sels[g], out=None if outs is None else outs[g][l])
                       for l in range(trace.wl.layers)]
    return gathered
