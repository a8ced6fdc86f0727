"""Randomised parity across the engine's paths at once (GPU).

Each seed draws a small workload with one to three layer groups, one of the two
policies (under PB-LRU one of the two placements of appended entries), a random
ring, one stream for every group or a stream per group (the library then runs
the groups' host-link launches one at a time), and per step and group a random
way to append: rows in
device memory or in host memory, with a per-call append limit small enough that
most appends run in several chunks (the plan / extract / place kernels) and the
rest in the one-workgroup path, through ula_append before ula_step or through
ula_append_step (which runs a small device-memory append in the step's first
launch). Each group's layers are gathered one call per layer, all in one
ula_gather_layers launch, or layer 0 alone and the rest in one launch, drawn per
step. Finished entries are released between steps.
After every step (and every release) each group's exported state must equal its
oracle's, and every gathered byte must equal the closed form of its row.
"""

import dataclasses

import numpy as np
import pytest

from gpu_harness import gather_layers_by, say
from synth import Trace, rows_for
from tracegen import padded_selections, release_plan, tiny_workload

pytestmark = pytest.mark.gpu


def _oracle(tr, g, policy, placement=0):
    from oracle.exact_lru_np import ExactLRUArrays
    from oracle.replay import initial_load, new_group
    if policy == 0:
        o = new_group(tr, full_data=True, placement="ring" if placement else "lowest")
        initial_load(o, tr, g)
    else:
        o = ExactLRUArrays(tr.N, tr.P, tr.H, tr.wl.ring)
        o.append(tr.initial_load_order())
    return o


def _same(st, ref, policy, where):
    for key in ("map", "gown", "hown"):
        assert np.array_equal(np.asarray(st[key]), np.asarray(ref[key])), f"{where}: {key} differs"
    assert st["flag"] == ref["flag"], f"{where}: flag"
    assert tuple(st["stats"]) == tuple(ref["stats"]), f"{where}: stats {st['stats']} vs {ref['stats']}"
    if policy == 0:
        assert np.array_equal(np.asarray(st["bitsets"]), np.asarray(ref["bitsets"])), f"{where}: bitsets"
        assert st["cur"] == ref["cur"], f"{where}: cur"
    else:
        assert np.array_equal(np.asarray(st["stamps"]), np.asarray(ref["stamps"])), f"{where}: stamps"


@pytest.mark.parametrize("seed", range(24))
def test_mixed_paths_random(seed):
    import torch
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device
    rng = np.random.default_rng([seed, 555])
    policy = int(rng.integers(0, 2))
    groups = int(rng.integers(1, 4))
    wl = tiny_workload(seed, steps=int(rng.integers(4, 11)))
    wl = dataclasses.replace(wl, groups=groups, appends=int(rng.integers(1, 4)), name=f"mixed{seed}")
    tr = Trace(wl)
    max_append = int(rng.integers(2, 6))
    placement = int(rng.integers(0, 2)) if policy == 0 else 0
    streams = [torch.cuda.Stream() for _ in range(groups)] if groups > 1 and rng.random() < 0.5 else None
    say(f"mixed {seed}: policy {policy} placement {placement} groups {groups} ring {wl.ring} "
        f"steps {tr.steps} N={tr.N} P={tr.P} H={tr.H} max_append={max_append} "
        f"streams {'per group' if streams else 'one'}")
    eng = engine_for(tr, max_append=max_append, policy=policy, placement=placement)
    rows_dev = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    try:
        initial_load(eng, tr, range(groups), rows_dev)
        ora = {g: _oracle(tr, g, policy, placement) for g in range(groups)}
        for g in range(groups):
            _same(eng.export_state(g), ora[g].export_state(), policy, f"group {g} after load")
        sels = {g: padded_selections(tr, g, seed + 7 * g) for g in range(groups)}
        plans = {g: release_plan(tr, sels[g], seed + 11 * g, frac=0.3) for g in range(groups)}
        for t in range(1, tr.steps + 1):
            app = tr.appends(t)
            for g in range(groups):
                sel = sels[g][t - 1]
                dsel = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
                combined = rng.random() < 0.5     # ula_append_step, else ula_append + ula_step
                rows = np.zeros((0, wl.layers, wl.row_bytes), np.uint8)
                if app.size:
                    host_rows = rng.random() < 0.5
                    rows = (rows_for(wl.seed, g, app, wl.layers, wl.row_bytes) if host_rows
                            else rows_dev(app, g))
                    if policy == 0:
                        ora[g].append(app, rows_for(wl.seed, g, app, wl.layers, wl.row_bytes))
                    else:
                        ora[g].append(app)
                gs = None
                if streams:   # the group's own stream, after the inputs made on the current one
                    gs = streams[g]
                    gs.wait_stream(torch.cuda.current_stream())
                if combined:
                    eng.append_step(g, app, rows, dsel, stream=gs)
                else:
                    if app.size:
                        eng.append(g, app, rows, stream=gs)
                    eng.step(g, dsel, stream=gs)
                mode = str(rng.choice(["layer", "all", "split"]))
                if gs is None:
                    outs = gather_layers_by(eng, g, wl.layers, dsel, mode)
                else:
                    with torch.cuda.stream(gs):
                        outs = gather_layers_by(eng, g, wl.layers, dsel, mode)
                ora[g].step(sel)
                eng.sync(stream=gs)
                _same(eng.export_state(g), ora[g].export_state(), policy, f"group {g} step {t}")
                flat = np.asarray(sel, dtype=np.int64).reshape(-1)
                want = np.zeros((flat.size, wl.layers, wl.row_bytes), np.uint8)
                ok = flat >= 0
                want[ok] = rows_for(wl.seed, g, flat[ok], wl.layers, wl.row_bytes)
                for l in range(wl.layers):
                    got = outs[l].cpu().numpy().reshape(flat.size, wl.row_bytes)
                    assert np.array_equal(got, want[:, l]), f"group {g} step {t} layer {l}: gathered rows differ"
                rel = plans[g].get(t, np.zeros(0, np.int32))
                if rel.size:
                    eng.release(g, rel)
                    ora[g].release(rel)
                    _same(eng.export_state(g), ora[g].export_state(), policy, f"group {g} release {t}")
    finally:
        eng.close()
