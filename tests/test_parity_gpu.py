"""Parity of the HIP engine with the CPU oracle (bit-exact), on the GPU.

Every case compares, after the initial load and after every step, the mapping
table, owners, bucket bitsets, current bucket, completion counter and step
statistics, and every gathered byte, with the oracle run on the same seeded
inputs. Sizes span several 1024-entry de-duplication blocks, several 2048-slot
summary spans and ragged tails.
"""

import dataclasses
import json
import os

import numpy as np
import pytest

from gpu_harness import assert_same_state, run_parity, say
from tracegen import padded_selections, tiny_workload
from synth import Trace, preset, rows_for, scaled

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_device_rows_match_numpy_rows():
    from synth.device import rows_device
    las = np.array([0, 1, 5, 4095, 123457, 2 ** 31 - 1], dtype=np.int32)
    for layers, rb, seed, g in [(1, 656, 0, 0), (3, 656, 7, 5), (2, 64, 255, 255)]:
        got = rows_device(las, layers, rb, seed, g).cpu().numpy()
        assert np.array_equal(got, rows_for(seed, g, las, layers, rb))


def test_worked_example_on_engine():
    import torch
    from serving_pb_lru_amd import Engine
    ex = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))
    z = ex["sizes"]
    eng = Engine(1, 1, 656, z["B"], z["N"], z["P"], z["H"], max_sets=1, max_k=4, max_append=3)
    try:
        las = np.array(ex["appends"], dtype=np.int32)
        eng.append(0, las, rows_for(0, 0, las, 1, 656))      # host-sourced rows, 3 chunks
        enc = lambda s: int(s[1:]) if s[0] == "G" else (0x80000000 | int(s[1:]))
        for s in ex["steps"]:
            sel = torch.tensor(s["sel"], dtype=torch.int32, device="cuda")
            eng.step(0, sel)
            out = eng.gather(0, 0, sel)
            eng.sync()
            st = eng.export_state(0)
            assert [int(x) for x in st["map"]] == [enc(x) for x in s["map"]]
            assert list(st["gown"]) == s["gown"] and list(st["hown"]) == s["hown"]
            assert int(st["bitsets"][0][0]) == s["free"] and int(st["bitsets"][1][0]) == s["cold"]
            assert [int(st["bitsets"][2 + b][0]) for b in range(2)] == s["ring"]
            assert st["cur"] == s["cur"] and list(st["stats"]) == s["stats"]
            o = out.cpu().numpy()
            for i, la in enumerate(s["gather"]):
                want = np.zeros(656, np.uint8) if la == -1 else rows_for(0, 0, [la], 1, 656)[0, 0]
                assert np.array_equal(o[0, i], want)
    finally:
        eng.close()


def test_tiny_4x4k_full_parity():
    run_parity(preset("tiny_4x4k"))


@pytest.mark.parametrize("seed", range(16))
def test_random_tiny_parity(seed):
    wl = tiny_workload(seed)
    tr = Trace(wl)
    run_parity(wl, selections={0: padded_selections(tr, 0, seed)}, max_append=7)


@pytest.mark.parametrize("seed", range(8))
def test_append_step_parity(seed):
    """ula_append_step (the step's appends in its first launch beside the tag pass)
    gives the same state and gathered bytes as ula_append then ula_step."""
    wl = dataclasses.replace(tiny_workload(seed), appends=1 + seed % 3)
    tr = Trace(wl)
    run_parity(wl, selections={0: padded_selections(tr, 0, seed)}, max_append=64, combined=True)


@pytest.mark.parametrize("name,factor,steps", [
    ("r16_64k_g1x3", 16, 8),
    ("spec3_r128_64k128k_g4", 32, 5),
])
def test_append_step_scaled_parity(name, factor, steps):
    wl = scaled(preset(name), factor)
    run_parity(wl, steps=steps, max_append=1 << 15, check_every=2, combined=True)


@pytest.mark.parametrize("mode", ["all", "split"])
@pytest.mark.parametrize("seed", range(6))
def test_gather_layers_parity(seed, mode):
    """ula_gather_layers (several layers of one selection in one launch) gives every
    layer's rows as the oracle gathers them: ragged selections with padding, two to
    four layers, both launch splits (all layers at once; layer 0, then the rest)."""
    wl = dataclasses.replace(tiny_workload(seed), layers=2 + seed % 3)
    tr = Trace(wl)
    run_parity(wl, selections={0: padded_selections(tr, 0, seed)}, max_append=7, gather_mode=mode)


@pytest.mark.parametrize("name,factor,steps,mode", [
    ("r16_64k_g1x3", 16, 6, "all"),
    ("r16_64k_g1x3", 16, 6, "split"),
    ("spec3_r128_64k128k_g4", 32, 4, "all"),
    ("evict_r256_128k_g2", 32, 5, "all"),
])
def test_gather_layers_scaled_parity(name, factor, steps, mode):
    wl = scaled(preset(name), factor)
    run_parity(wl, steps=steps, max_append=1 << 15, check_every=2, combined=True, gather_mode=mode)


@pytest.mark.parametrize("k,layers", [(32_768, 2), (65_536, 2), (65_537, 2), (43_690, 3), (43_691, 3),
                                      (32_767, 4), (70_001, 2)])
def test_gather_layers_tilings_parity(k, layers):
    """Gathers on every side of the tiling switches, with partial last blocks, against
    the oracle: one-layer launches up to 65,536 rows and multi-layer launches up to
    131,072 row-layers take the small tilings (32 rows for two layers, 16 for three or
    more: 65,536 x 2, 43,690 x 3 and 32,767 x 4 are small, 65,537 x 2 and 43,691 x 3
    the first large ones), and the one-layer launch of layer 0 beside them (32,767,
    32,768, 43,690 and 65,536 rows small, 65,537 and 70,001 large)."""
    from synth.configs import Workload
    wl = Workload(name=f"layers{k}x{layers}", requests=1, ctx_fixed=200_000, ctx_range=None,
                  sets_per_request=1, draft_keep=0.0, groups=1, layers=layers, k=k, pool_frac=0.0,
                  pool_slots=100_000, ring=4, steps=3, appends=1, overlap=0.85, p_recent=0.7,
                  window=4096, row_bytes=64, seed=9)
    run_parity(wl, max_append=1 << 12, gather_mode="all")
    run_parity(wl, max_append=1 << 12, gather_mode="split")


def test_gather_layers_every_window():
    """Every window (layer0, n_layers) of a four-layer group, including a selection
    with padding and repeated entries, equals the per-layer gathers of its layers, and
    bytes outside the window's buffers are left alone."""
    import torch
    from synth.device import rows_device
    from serving_pb_lru_amd.replay import engine_for, initial_load
    wl = dataclasses.replace(tiny_workload(3), layers=4, name="window4")
    tr = Trace(wl, 3)
    eng = engine_for(tr, max_append=64)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    try:
        initial_load(eng, tr, [0], rows)
        sels = list(padded_selections(tr, 0, 3, frac=0.2))
        for t in range(1, tr.steps + 1):
            app = tr.appends(t)
            eng.append_step(0, app, rows(app, 0), torch.from_numpy(sels[t - 1]).cuda())
        sel = sels[-1].copy()
        sel[0, -1] = sel[0, 0]                       # a repeated entry
        dsel = torch.from_numpy(np.ascontiguousarray(sel)).cuda()
        want = [eng.gather(0, l, dsel).cpu().numpy() for l in range(wl.layers)]
        for l0 in range(wl.layers):
            for nl in range(1, wl.layers - l0 + 1):
                buf = torch.full((nl + 1, *sel.shape, wl.row_bytes), 0xA5, dtype=torch.uint8, device="cuda")
                eng.gather_layers(0, l0, nl, dsel, out=buf)
                got = buf.cpu().numpy()
                for i in range(nl):
                    assert np.array_equal(got[i], want[l0 + i]), (l0, nl, i)
                assert (got[nl] == 0xA5).all(), (l0, nl)
        eng.sync()
    finally:
        eng.close()


@pytest.mark.parametrize("appends,pool_frac", [(1, 0.5), (2, 0.0)])
def test_append_step_many_appends_parity(appends, pool_frac):
    """ula_append_step with more appends per step (300 and 600) than the step's first
    launch takes (256): they run as ula_append does, before the step; with room on the
    GPU and with a full GPU pool (appends into host slots)."""
    from synth.configs import Workload
    wl = Workload(name=f"many_appends{appends}", requests=300, ctx_fixed=2048, ctx_range=None,
                  sets_per_request=1, draft_keep=0.0, groups=1, layers=2, k=64, pool_frac=pool_frac,
                  pool_slots=None if pool_frac else 40_000, ring=4, steps=4, appends=appends, overlap=0.8,
                  p_recent=0.7, window=256, row_bytes=64, seed=3)
    run_parity(wl, max_append=1024, combined=True)


@pytest.mark.parametrize("ring", [1, 2, 9, 64])   # 64: the longest ring the engine takes
def test_ring_lengths_parity(ring):
    wl = dataclasses.replace(preset("tiny_4x4k"), ring=ring, name=f"tiny_ring{ring}")
    run_parity(wl)


@pytest.mark.parametrize("row_bytes,layers", [(16, 1), (16, 3), (1024, 2)])
def test_row_sizes_parity(row_bytes, layers):
    """The smallest row (one 16-byte piece), a three-layer slot of such rows, and the
    largest row the synthetic generator makes (64 pieces): the gather, swap, prefetch,
    write-back and append loops with unusual piece counts per row and per slot."""
    base = tiny_workload(5)
    wl = dataclasses.replace(base, row_bytes=row_bytes, layers=layers, name=f"rows{row_bytes}x{layers}")
    tr = Trace(wl)
    run_parity(wl, selections={0: padded_selections(tr, 0, 5)}, max_append=7)


@pytest.mark.parametrize("name,factor,steps,check_every", [
    ("r16_64k_g1x3", 16, 10, 1),
    ("r16_64k_g1x3", 16, 10, 4),
    ("r64_64k128k_g24x3", 32, 5, 1),
    ("spec3_r128_64k128k_g4", 32, 6, 1),
    ("spec3_r128_64k128k_g4", 32, 6, 100),
    ("evict_r256_128k_g2", 32, 8, 1),
    ("evict_r256_128k_g2", 32, 8, 3),
    ("evict_r256_128k_g2_ctl98", 32, 6, 1),
    # ~19.5 MB each way per group step: the link moves both directions in every
    # link workgroup (4 MB and more)
    ("evict_r256_128k_g2", 8, 4, 1),
])
def test_scaled_workload_parity(name, factor, steps, check_every):
    wl = scaled(preset(name), factor)
    groups = None if wl.groups <= 4 else [0, 7, 23]
    run_parity(wl, steps=steps, groups=groups, max_append=1 << 15, check_every=check_every)


def test_large_gather_ragged_parity():
    """A selection of 70,001 entries: the large-gather tiling (above 65,536 rows) with a
    partial last block, and a lookup with a partial last workgroup, against the oracle."""
    from synth.configs import Workload
    wl = Workload(name="ragged70001", requests=1, ctx_fixed=200_000, ctx_range=None, sets_per_request=1,
                  draft_keep=0.0, groups=1, layers=2, k=70_001, pool_frac=0.0, pool_slots=100_000, ring=4,
                  steps=3, appends=1, overlap=0.85, p_recent=0.7, window=4096, row_bytes=64, seed=9)
    ora = run_parity(wl, max_append=1 << 12)
    assert ora[0].last.misses > 0


@pytest.mark.parametrize("schedule", ["group", "two+gather"])
@pytest.mark.parametrize("policy", [0, 1], ids=["pblru", "lru"])
def test_groups_on_separate_streams(policy, schedule):
    """Layer groups are independent and may be driven on different streams: each
    group's appends, steps and gathers go to a stream of its own (schedule
    "group"), or the groups' appends and steps alternate over two streams and
    every gather runs on a third, after an event its step recorded, with each
    group's next append waiting for an event after its gathers (schedule
    "two+gather", bench.py's for more than two groups); no other
    synchronisation between the groups. Every group matches its own oracle
    (every gathered byte of every step, and the state after the last step)."""
    import torch
    from oracle.exact_lru_np import ExactLRUArrays
    from oracle.replay import initial_load as oracle_load, new_group
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device
    wl = scaled(preset("spec3_r128_64k128k_g4"), 32)
    tr = Trace(wl, 6)
    G = wl.groups
    say(f"separate streams {wl.name} policy {policy} schedule {schedule}: groups={G} steps={tr.steps}")
    eng = engine_for(tr, max_append=1 << 15, policy=policy)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    try:
        initial_load(eng, tr, range(G), rows)
        sels = {g: list(tr.selections(g)) for g in range(G)}
        dsel = {g: [torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda() for x in sels[g]]
                for g in range(G)}
        app_rows = {(g, t): rows(tr.appends(t), g) for g in range(G) for t in range(1, tr.steps + 1)
                    if tr.appends(t).size}
        torch.cuda.synchronize()
        if schedule == "group":
            streams = [torch.cuda.Stream() for _ in range(G)]
            gstreams = streams
        else:
            pair = [torch.cuda.Stream(), torch.cuda.Stream()]
            streams = [pair[g % 2] for g in range(G)]
            gather_stream = torch.cuda.Stream()
            gstreams = [gather_stream] * G
        step_done = [torch.cuda.Event() for _ in range(G)]
        gathers_done = [torch.cuda.Event() for _ in range(G)]
        outs = {}
        for t in range(1, tr.steps + 1):
            app = tr.appends(t)
            for g in range(G):
                if schedule != "group":
                    streams[g].wait_event(gathers_done[g])
                if app.size:
                    eng.append(g, app, app_rows[(g, t)], stream=streams[g])
                eng.step(g, dsel[g][t - 1], stream=streams[g])
                if schedule != "group":
                    step_done[g].record(streams[g])
                    gstreams[g].wait_event(step_done[g])
                outs[(g, t)] = [eng.gather(g, l, dsel[g][t - 1], stream=gstreams[g]) for l in range(wl.layers)]
                if schedule != "group":
                    gathers_done[g].record(gstreams[g])
        torch.cuda.synchronize()
        eng.sync()
        for g in range(G):
            if policy == 0:
                ora = new_group(tr, full_data=True)
                oracle_load(ora, tr, g)
            else:
                ora = ExactLRUArrays(tr.N, tr.P, tr.H, wl.ring)
                ora.append(tr.initial_load_order())
            for t in range(1, tr.steps + 1):
                app = tr.appends(t)
                sel = sels[g][t - 1]
                if policy == 0:
                    ora.append(app, rows_for(wl.seed, g, app, wl.layers, wl.row_bytes))
                    ora.step(sel)
                else:
                    ora.append(app)
                    ora.step(sel)
                for l in range(wl.layers):
                    got = outs[(g, t)][l].cpu().numpy()
                    flat = sel.reshape(-1)
                    want = np.zeros((flat.size, wl.row_bytes), np.uint8)
                    ok = flat >= 0
                    want[ok] = rows_for(wl.seed, g, flat[ok], wl.layers, wl.row_bytes)[:, l]
                    assert np.array_equal(got.reshape(flat.size, wl.row_bytes), want), \
                        f"group {g} step {t} layer {l}: gathered rows differ"
            st = eng.export_state(g)
            ref = ora.export_state()
            for key in ("map", "gown", "hown"):
                assert np.array_equal(np.asarray(st[key]), np.asarray(ref[key])), f"group {g}: {key} differs"
            assert st["flag"] == ref["flag"] and tuple(st["stats"]) == tuple(ref["stats"]), f"group {g}"
            if policy == 0:
                assert np.array_equal(np.asarray(st["bitsets"]), np.asarray(ref["bitsets"])), f"group {g}: bitsets"
            else:
                assert np.array_equal(np.asarray(st["stamps"]), np.asarray(ref["stamps"])), f"group {g}: stamps"
    finally:
        eng.close()


def _pingpong():
    """One request of 64 positions, a pool of 8 slots, 2 ring buckets and k = 8:
    alternating disjoint sets miss every entry and evict the previous set, so
    most misses ask for rows evicted by the step just before."""
    from synth.configs import Workload
    wl = Workload(name="pingpong", requests=1, ctx_fixed=64, ctx_range=None, sets_per_request=1,
                  draft_keep=0.0, groups=1, layers=2, k=8, pool_frac=0.0, pool_slots=8, ring=2,
                  steps=12, appends=0, overlap=0.0, p_recent=0.0, window=8, row_bytes=64, seed=3)
    A, B, C = (np.arange(8 * i, 8 * i + 8, dtype=np.int32)[None, :] for i in range(3))
    mix = np.concatenate([A[:, :4], B[:, 4:]], axis=1)
    return wl, [A, B, A, B, C, A, B, mix, C, A, B, A]


@pytest.mark.parametrize("check_every", [1, 2, 5, 100])
def test_evicted_rows_missed_next_step(check_every):
    wl, sels = _pingpong()
    ora = run_parity(wl, selections={0: sels}, check_every=check_every)
    assert ora[0].last.as_tuple()[2:4] == (8, 8)   # the last step still swaps every entry


def test_pool_holds_everything_parity():
    wl = dataclasses.replace(preset("tiny_4x4k"), name="tiny_all_gpu")
    tr = Trace(wl)
    wl = dataclasses.replace(wl, pool_slots=tr.N)
    run_parity(wl)


@pytest.mark.parametrize("seed", range(8))
def test_release_parity_random(seed):
    """Finished entries released between steps (their GPU slots join the free set,
    their host slots the free host set); later misses take the freed GPU slots first
    and appends reuse freed slots. State and gathered bytes match the oracle."""
    from tracegen import release_plan
    wl = tiny_workload(seed, steps=10)
    tr = Trace(wl)
    sels = padded_selections(tr, 0, seed)
    ora = run_parity(wl, selections={0: sels}, max_append=7, check_every=1 if seed % 2 else 3,
                     releases=release_plan(tr, sels, seed, frac=0.4))
    assert ora[0].flag == tr.steps


@pytest.mark.parametrize("name,factor,steps", [
    ("r16_64k_g1x3", 16, 8),
    ("evict_r256_128k_g2", 32, 6),
])
def test_release_parity_scaled(name, factor, steps):
    from tracegen import release_plan
    wl = scaled(preset(name), factor)
    tr = Trace(wl, steps)
    sels = {g: list(tr.selections(g)) for g in range(wl.groups)}
    # one release plan for every group: addresses no group's later steps select
    merged = [np.concatenate([sels[g][t].reshape(-1) for g in sels]) for t in range(steps)]
    plan = release_plan(tr, merged, 7, frac=0.3)
    run_parity(wl, steps=steps, selections=sels, max_append=1 << 15, check_every=2, releases=plan)
