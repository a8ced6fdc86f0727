"""Drive a decode trace through the engine (initial load, then per step: the
step's appends and the step in one call, then the group's layers: the first
gathered alone, the later ones in one launch). Used by the GPU tests, smoke()
and bench.py.

The trace object supplies the addresses (initial_load_order, appends(t),
selections(g)); `rows(las, g)` supplies the appended rows as a CUDA tensor.
"""

from __future__ import annotations

import numpy as np

from .ula import Engine

LOAD_CHUNK = 1 << 18


def engine_for(trace, max_append: int = 1 << 16, policy: int = 0, placement: int = 0) -> Engine:
    wl = trace.wl
    return Engine(num_groups=wl.groups, layers=wl.layers, row_bytes=wl.row_bytes, ring=wl.ring,
                  logical_capacity=trace.N, gpu_slots=trace.P, host_slots=trace.H,
                  max_sets=trace.n_sets, max_k=trace.k, max_append=max_append, policy=policy,
                  placement=placement)


def initial_load(eng: Engine, trace, groups, rows) -> None:
    order = trace.initial_load_order()
    for g in groups:
        for s in range(0, order.size, LOAD_CHUNK):
            las = order[s:s + LOAD_CHUNK]
            eng.append(g, las, rows(las, g))


def step_all(eng: Engine, trace, t: int, sels, groups, rows):
    """Step t for the given groups. sels[g]: CUDA int32 [n_sets][k]. Returns, per
    group, one gathered tensor per layer."""
    app = trace.appends(t)
    layers = trace.wl.layers
    gathered = {}
    for g in groups:
        eng.append_step(g, app, rows(app, g), sels[g])
        outs = [eng.gather(g, 0, sels[g])]
        if layers > 1:
            outs += list(eng.gather_layers(g, 1, layers - 1, sels[g]))
        gathered[g] = outs
    return gathered
