"""Gathers of selections other than the step's own (GPU).

A step resolves its own selection entry by entry; a gather reads that
resolution where its entry matches and goes through the mapping table
everywhere else (UlaCache summary, section 3: a reader sees every GPU-resident
entry at its slot once the step has signalled). Here, after each step, the
gathered selection is a permutation of the step's (same size, so the one-layer
gather takes its non-temporal loads while no entry matches its position), a
prefix of it, the step's selection followed by other resident entries, and a
mix with other resident entries and padding. Every gathered byte must equal
the selected entries' rows (zeros for padding), and the state after the last
step must equal the oracle's.
"""

import dataclasses

import numpy as np
import pytest

from gpu_harness import assert_same_state, say
from oracle.replay import initial_load as oracle_load, new_group
from synth import Trace, preset, rows_for

pytestmark = pytest.mark.gpu


def _want(wl, sel, layer):
    flat = np.asarray(sel).reshape(-1)
    out = np.zeros((flat.size, wl.row_bytes), np.uint8)
    ok = flat >= 0
    if ok.any():
        out[ok] = rows_for(wl.seed, 0, flat[ok], wl.layers, wl.row_bytes)[:, layer]
    return out


def _variants(sel, resident, rng):
    """Other selections to gather after a step that selected `sel`; `resident`
    holds GPU-resident addresses that the step did not select."""
    flat = sel.reshape(-1)
    n = flat.size
    perm = flat[rng.permutation(n)].reshape(sel.shape)
    prefix = flat[: n // 2 + 1].reshape(1, -1)
    extra = rng.choice(resident, size=min(sel.shape[1], resident.size), replace=False)
    longer = np.concatenate([flat, extra]).reshape(2, -1)
    mixed = flat.copy()
    pos = rng.choice(n, size=n // 3, replace=False)
    mixed[pos] = rng.choice(resident, size=pos.size, replace=True)
    mixed[rng.choice(n, size=n // 7, replace=False)] = -1
    return {"permuted": perm, "prefix": prefix, "longer": longer, "mixed": mixed.reshape(sel.shape)}


@pytest.mark.parametrize("repeats", [False, True], ids=["distinct", "repeats"])
@pytest.mark.parametrize("layers", [1, 2])
def test_gather_other_selections(layers, repeats):
    """With `repeats`, the second request's first 64 entries repeat the first's
    (entries that several requests select), so no gather after that step takes
    the non-temporal loads."""
    import torch
    from serving_pb_lru_amd import Engine
    from serving_pb_lru_amd.replay import initial_load
    from synth.device import rows_device

    wl = dataclasses.replace(preset("tiny_4x4k"), layers=layers, name=f"tiny_l{layers}")
    tr = Trace(wl, 6)
    say(f"other selections: layers={layers} repeats={repeats} steps={tr.steps} N={tr.N} P={tr.P}")
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    # rows up to four times the step's width, for the longer selections
    eng = Engine(1, wl.layers, wl.row_bytes, wl.ring, tr.N, tr.P, tr.H, max_sets=tr.n_sets,
                 max_k=4 * tr.k, max_append=4096)
    ora = new_group(tr, full_data=False)
    oracle_load(ora, tr, 0)
    rng = np.random.default_rng(7 + layers)
    try:
        initial_load(eng, tr, [0], rows)
        for t, sel in enumerate(tr.selections(0), start=1):
            if repeats:
                sel = sel.copy()
                sel[1, :64] = sel[0, :64]
            app = tr.appends(t)
            d = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
            eng.append_step(0, app, rows(app, 0), d)
            eng.sync()
            ora.append(app, None)
            ora.step(sel)
            st = eng.export_state(0)
            m = np.asarray(st["map"], dtype=np.uint32)
            flat = sel.reshape(-1)
            distinct = np.unique(flat[flat >= 0]).size == (flat >= 0).sum()
            assert distinct != repeats, "the step's selection repeats entries only when asked to"
            on_gpu = np.flatnonzero(m & 0x80000000 == 0).astype(np.int32)
            resident = np.setdiff1d(on_gpu, flat)
            assert resident.size, "no other resident entry to gather"
            for kind, other in _variants(sel, resident, rng).items():
                o = torch.from_numpy(np.ascontiguousarray(other, dtype=np.int32)).cuda()
                got = [eng.gather(0, l, o) for l in range(layers)]
                if layers > 1:
                    got_all = eng.gather_layers(0, 0, layers, o)
                eng.sync()
                for l in range(layers):
                    want = _want(wl, other, l)
                    g1 = got[l].cpu().numpy().reshape(want.shape)
                    assert np.array_equal(g1, want), f"step {t} {kind} layer {l}: ula_gather rows differ"
                    if layers > 1:
                        g2 = got_all[l].cpu().numpy().reshape(want.shape)
                        assert np.array_equal(g2, want), f"step {t} {kind} layer {l}: ula_gather_layers"
        assert_same_state(eng.export_state(0), ora.export_state(), "after the last step")
    finally:
        eng.close()
