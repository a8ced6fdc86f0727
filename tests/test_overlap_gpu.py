"""A group's next step may be enqueued while its previous step's gathers still run
on another stream, with nothing ordering the two: the library makes only the
launches that move rows out of GPU slots (the next step's swap, appends under the
second placement, releases) wait for those gathers, by events; the next step's
lookup, marking and host-link transfers run beside them, each step resolving its
selection into one of two buffers by step parity (UlaCache summary, section 3:
readers see the moved rows only after the signal, and never half-moved ones).

Here every step (with its appends) goes to one of the step streams, every gather
to a separate gather stream after an event its step recorded, and releases go to
the step stream between steps, all enqueued without host synchronisation. Every
gathered byte of every step must equal the rows of the selected entries (zeros
for padding), and after the last step the state must equal the oracle's.
"""

import dataclasses

import numpy as np
import pytest

from gpu_harness import assert_same_state, say
from synth import Trace, preset, rows_for, scaled
from tracegen import release_plan, tiny_workload

pytestmark = pytest.mark.gpu


def _expected(wl, g, sel, layer):
    flat = np.asarray(sel).reshape(-1)
    want = np.zeros((flat.size, wl.row_bytes), np.uint8)
    ok = flat >= 0
    if ok.any():
        want[ok] = rows_for(wl.seed, g, flat[ok], wl.layers, wl.row_bytes)[:, layer]
    return want


def run_overlapped(wl, steps, policy=0, placement=0, release_frac=0.0, split=False, step_streams=1,
                   seed=0, release_side=False):
    """release_side: each release goes to a stream of its own, ordered after its
    group's step by an event, and the group's next step after the release by
    another (the library alone orders the release after the step's gathers)."""
    import torch
    from oracle.exact_lru_np import ExactLRUArrays
    from oracle.replay import initial_load as oracle_load, new_group
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device

    tr = Trace(wl, steps)
    G = wl.groups
    L = wl.layers
    say(f"overlapped {wl.name}: groups={G} layers={L} steps={tr.steps} policy={policy} "
        f"placement={placement} releases={release_frac} split={split} step_streams={step_streams} "
        f"release_side={release_side}")
    eng = engine_for(tr, max_append=1 << 15, policy=policy, placement=placement)
    rows = lambda las, g: rows_device(las, L, wl.row_bytes, wl.seed, g)
    try:
        initial_load(eng, tr, range(G), rows)
        sels = {g: list(tr.selections(g)) for g in range(G)}
        dsel = {g: [torch.from_numpy(np.ascontiguousarray(s, dtype=np.int32)).cuda() for s in sels[g]]
                for g in range(G)}
        app_rows = {(g, t): rows(tr.appends(t), g) for g in range(G) for t in range(1, tr.steps + 1)}
        rel = {g: (release_plan(tr, sels[g], seed + g, frac=release_frac) if release_frac else {})
               for g in range(G)}
        # every step's output buffers up front, so nothing is freed while in use
        outs = {(g, t): torch.empty((L, tr.n_sets, tr.k, wl.row_bytes), dtype=torch.uint8, device="cuda")
                for g in range(G) for t in range(1, tr.steps + 1)}
        torch.cuda.synchronize()
        step_s = [torch.cuda.Stream() for _ in range(step_streams)]
        gather_s = torch.cuda.Stream()
        rel_s = torch.cuda.Stream()
        done = [torch.cuda.Event() for _ in range(G)]
        for t in range(1, tr.steps + 1):
            app = tr.appends(t)
            for g in range(G):
                s = step_s[g % step_streams]
                eng.append_step(g, app, app_rows[(g, t)], dsel[g][t - 1], stream=s)
                done[g].record(s)
                gather_s.wait_event(done[g])
                o = outs[(g, t)]
                if split:
                    eng.gather(g, 0, dsel[g][t - 1], out=o[0], stream=gather_s)
                    if L > 1:
                        eng.gather_layers(g, 1, L - 1, dsel[g][t - 1], out=o[1:], stream=gather_s)
                else:
                    for l in range(L):
                        eng.gather(g, l, dsel[g][t - 1], out=o[l], stream=gather_s)
                if t in rel[g] and rel[g][t].size:
                    if release_side:
                        rel_s.wait_event(done[g])
                        eng.release(g, rel[g][t], stream=rel_s)
                        back = torch.cuda.Event()
                        back.record(rel_s)
                        s.wait_event(back)
                    else:
                        eng.release(g, rel[g][t], stream=s)
        torch.cuda.synchronize()
        eng.sync()
        for g in range(G):
            if policy == 0:
                ora = new_group(tr, full_data=False, placement="ring" if placement else "lowest")
                oracle_load(ora, tr, g)
            else:
                ora = ExactLRUArrays(tr.N, tr.P, tr.H, wl.ring)
                ora.append(tr.initial_load_order())
            for t in range(1, tr.steps + 1):
                sel = sels[g][t - 1]
                if policy == 0:
                    ora.append(tr.appends(t), None)
                else:
                    ora.append(tr.appends(t))
                ora.step(sel)
                got = outs[(g, t)].cpu().numpy()
                for l in range(L):
                    want = _expected(wl, g, sel, l)
                    if not np.array_equal(got[l].reshape(want.shape), want):
                        bad = np.argwhere((got[l].reshape(want.shape) != want).any(axis=-1))
                        raise AssertionError(f"group {g} step {t} layer {l}: gathered rows differ at "
                                             f"{len(bad)} rows, first {bad[:5].ravel().tolist()}")
                if t in rel[g] and rel[g][t].size:
                    ora.release(rel[g][t])
            st = eng.export_state(g)
            ref = ora.export_state()
            if policy == 0:
                assert_same_state(st, ref, f"group {g} after the last step")
            else:
                for key in ("map", "gown", "hown", "stamps"):
                    assert np.array_equal(np.asarray(st[key]), np.asarray(ref[key])), f"group {g}: {key}"
                assert st["flag"] == ref["flag"] and tuple(st["stats"]) == tuple(ref["stats"]), f"group {g}"
    finally:
        eng.close()


@pytest.mark.parametrize("policy", [0, 1], ids=["pblru", "lru"])
def test_overlap_four_groups_two_step_streams(policy):
    """bench.py's schedule for more than two groups, without the explicit wait of
    each step for its group's gathers."""
    run_overlapped(scaled(preset("spec3_r128_64k128k_g4"), 32), 6, policy=policy, step_streams=2)


@pytest.mark.parametrize("split", [False, True], ids=["per_layer", "split"])
def test_overlap_one_group_three_layers(split):
    run_overlapped(scaled(preset("r16_64k_g1x3"), 16), 8, split=split)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("placement", [0, 1], ids=["lowest", "ring"])
def test_overlap_random_with_releases(seed, placement):
    """Evicting appends (second placement) and releases between the steps: both
    move rows out of GPU slots that the previous step's gathers may still read."""
    wl = tiny_workload(seed + 300, steps=10)
    wl = dataclasses.replace(wl, appends=1 + seed % 3, groups=1 + seed % 2, name=f"ovl{seed}")
    run_overlapped(wl, None, placement=placement, release_frac=0.3, seed=seed,
                   step_streams=1 + seed % 2)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("placement", [0, 1], ids=["lowest", "ring"])
def test_overlap_releases_on_their_own_stream(seed, placement):
    """Releases on a third stream: ordered after the step and before the next
    step by the caller's events, after the step's gathers by the library."""
    wl = tiny_workload(seed + 500, steps=10)
    wl = dataclasses.replace(wl, appends=1 + seed % 3, groups=1 + seed % 2, name=f"ovl_rel{seed}")
    run_overlapped(wl, None, placement=placement, release_frac=0.4, seed=seed, release_side=True)


@pytest.mark.parametrize("seed", range(4))
def test_overlap_random_exact_lru_with_releases(seed):
    wl = tiny_workload(seed + 400, steps=10)
    wl = dataclasses.replace(wl, appends=1 + seed % 2, name=f"ovl_lru{seed}")
    run_overlapped(wl, None, policy=1, release_frac=0.3, seed=seed)


@pytest.mark.parametrize("placement", [0, 1], ids=["lowest", "ring"])
def test_overlap_bulk_appends(placement):
    """300 appends per step, more than the step's first launch takes: they go
    through the bulk append kernels (ula_append inside ula_append_step), which
    under the second placement must also wait for the previous step's gathers."""
    from synth.configs import Workload
    wl = Workload(name=f"ovl_bulk{placement}", requests=300, ctx_fixed=2048, ctx_range=None,
                  sets_per_request=1, draft_keep=0.0, groups=1, layers=2, k=64, pool_frac=0.0,
                  pool_slots=40_000, ring=4, steps=5, appends=1, overlap=0.8, p_recent=0.7,
                  window=256, row_bytes=64, seed=5)
    run_overlapped(wl, None, placement=placement, release_frac=0.2, seed=placement)
