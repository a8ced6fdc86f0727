"""Exact-LRU policy of the HIP engine against the oracle's brute-force exact LRU (GPU).

UlaCache summary (paper-daily.com), sections 3-4: textbook LRU, a last-use stamp
on every slot and a pass over the whole pool to pick victims, is the policy
PB-LRU is compared against. The engine's exact-LRU mode (select passes over the
whole pool, slot-ordered emission, stable radix sort) must pick the same
victims in the same order as the oracle's plain scan-and-sort, so after every
step the mapping table, owners, timestamps, free set, counter and statistics
agree bit for bit, and every gathered byte equals its closed form.
"""

import dataclasses

import numpy as np
import pytest

from gpu_harness import say
from oracle.exact_lru import ExactLRUGroup
from synth import Trace, preset, rows_for, scaled
from tracegen import padded_selections, tiny_workload

pytestmark = pytest.mark.gpu


def _lru_state(lru: ExactLRUGroup, P: int) -> dict:
    W = (P + 31) // 32
    free = np.zeros(W * 32, dtype=bool)
    free[list(lru.free_gpu)] = True
    words = np.packbits(free.reshape(W, 32)[:, ::-1], axis=1, bitorder="big").view(">u4").reshape(W)
    stamps = np.array([lru.stamp[s] if lru.gown[s] != -1 else 0 for s in range(P)], dtype=np.int32)
    return dict(map=np.array(lru.map_array(), dtype=np.uint32), gown=np.array(lru.gown, dtype=np.int32),
                hown=np.array(lru.hown, dtype=np.int32), free=words.astype(np.uint32), stamps=stamps,
                flag=lru.t, stats=lru.last)


def _compare(st: dict, ref: dict, where: str) -> None:
    for key in ("map", "gown", "hown", "stamps"):
        a, b = np.asarray(st[key]), np.asarray(ref[key])
        if not np.array_equal(a, b):
            bad = np.flatnonzero(a != b)
            raise AssertionError(f"{where}: {key} differs at {bad.size} places, first {bad[:5]}: "
                                 f"engine {a[bad[:5]]} oracle {b[bad[:5]]}")
    assert np.array_equal(st["bitsets"][0], ref["free"]), f"{where}: free set differs"
    assert not st["bitsets"][1:].any(), f"{where}: exact LRU keeps no buckets"
    assert st["flag"] == ref["flag"], f"{where}: flag"
    if ref["stats"] is not None:
        assert tuple(st["stats"]) == tuple(ref["stats"]), f"{where}: stats {st['stats']} vs {ref['stats']}"


def run_lru_parity(wl, steps=None, selections=None, check_every=1, max_append=4096, groups=None,
                   releases=None):
    """Every group of one engine against its own oracle, steps interleaved group by group."""
    import torch
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device
    tr = Trace(wl, steps)
    groups = [0] if groups is None else groups
    say(f"lru parity {wl.name}: N={tr.N} P={tr.P} H={tr.H} steps={tr.steps} groups={groups}")
    eng = engine_for(tr, max_append=max_append, policy=1)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    lru = {g: ExactLRUGroup(tr.N, tr.P, tr.H) for g in groups}
    try:
        initial_load(eng, tr, groups, rows)
        for g in groups:
            lru[g].append(tr.initial_load_order())
            _compare(eng.export_state(g), _lru_state(lru[g], tr.P), f"group {g} after load")
        sels = {g: (iter(selections) if selections is not None else tr.selections(g)) for g in groups}
        for t in range(1, tr.steps + 1):
            app = tr.appends(t)
            for g in groups:
                sel = next(sels[g])
                if app.size:
                    eng.append(g, app, rows(app, g))
                    lru[g].append(app)
                dsel = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
                eng.step(g, dsel)
                outs = [eng.gather(g, l, dsel) for l in range(wl.layers)]
                eng.sync()
                lru[g].step(sel)
                if t % check_every == 0 or t == tr.steps:
                    _compare(eng.export_state(g), _lru_state(lru[g], tr.P), f"group {g} step {t}")
                flat = np.asarray(sel, dtype=np.int32).reshape(-1)
                want = rows_for(wl.seed, g, np.where(flat < 0, 0, flat), wl.layers, wl.row_bytes)
                want[flat < 0] = 0
                for l in range(wl.layers):
                    got = outs[l].cpu().numpy().reshape(flat.size, wl.row_bytes)
                    assert np.array_equal(got, want[:, l]), f"group {g} step {t} layer {l}: gathered rows differ"
                if releases is not None and t in releases and releases[t].size:
                    eng.release(g, releases[t])
                    lru[g].release(releases[t])
                    _compare(eng.export_state(g), _lru_state(lru[g], tr.P), f"group {g} after release {t}")
        known = np.concatenate([tr.initial_load_order()] + [tr.appends(t) for t in range(1, tr.steps + 1)])
        if releases is not None:
            known = np.setdiff1d(known, np.concatenate([np.zeros(0, np.int32)] + list(releases.values())))
        for g in groups:
            assert np.array_equal(eng.read_rows(g, known), rows_for(wl.seed, g, known, wl.layers, wl.row_bytes))
        return lru[groups[0]]
    finally:
        eng.close()


def test_lru_tiny_4x4k():
    run_lru_parity(preset("tiny_4x4k"))


@pytest.mark.parametrize("seed", range(10))
def test_lru_random_tiny(seed):
    # pools close to the step's working set: old steps' slots are evicted, so the
    # victims mix several timestamps and the radix sort orders them
    wl = tiny_workload(seed, steps=12)
    tr = Trace(wl)
    run_lru_parity(wl, selections=padded_selections(tr, 0, seed), max_append=7,
                   check_every=1 if seed % 2 else 3)


def test_lru_long_trace_two_sort_passes():
    # past step 255 the keys need two 8-bit sort passes; a pool of twice one
    # step's selection makes most steps' victims span several timestamps (on the
    # oracle: 293 of 300 steps, 42 of them past step 255)
    wl = tiny_workload(2, steps=300, sets=1, layers=1)
    wl = dataclasses.replace(wl, pool_slots=2 * wl.requests * wl.k, name="long300")
    lru = run_lru_parity(wl, check_every=50)
    assert lru.t == 300


def test_lru_long_trace_two_select_passes():
    # keys never exceed the step number, so the selection runs one 10-bit pass up
    # to step 1023 and two from step 1024 (bits 10-20, then 0-9): a 1100-step
    # trace crosses over, with state checked every 25 steps around the crossing
    wl = tiny_workload(2, steps=1100, sets=1, layers=1)
    wl = dataclasses.replace(wl, pool_slots=2 * wl.requests * wl.k, name="long1100")
    lru = run_lru_parity(wl, check_every=25)
    assert lru.t == 1100


@pytest.mark.parametrize("name,factor,steps", [
    ("r16_64k_g1x3", 16, 8),
    ("evict_r256_128k_g2", 64, 6),
    ("spec3_r128_64k128k_g4", 64, 4),
    ("evict_r256_128k_g2", 8, 4),   # both link directions in every link workgroup
])
def test_lru_scaled(name, factor, steps):
    wl = scaled(preset(name), factor)
    run_lru_parity(wl, steps=steps, check_every=2, max_append=1 << 15, groups=list(range(wl.groups)))


def test_lru_equals_long_ring_pblru_on_gpu():
    """With a ring longer than the trace PB-LRU never folds and equals exact LRU:
    the two engine modes must end in the same mapping table and owners."""
    import torch
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device
    wl = dataclasses.replace(preset("tiny_4x4k"), ring=9, name="tiny_ring9")
    tr = Trace(wl)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    engs = [engine_for(tr, policy=p) for p in (0, 1)]
    try:
        for e in engs:
            initial_load(e, tr, [0], rows)
        sels = tr.selections(0)
        for t in range(1, tr.steps + 1):
            sel = torch.from_numpy(next(sels)).cuda()
            app = tr.appends(t)
            for e in engs:
                if app.size:
                    e.append(0, app, rows(app, 0))
                e.step(0, sel)
        a, b = (e.export_state(0) for e in engs)
        for key in ("map", "gown", "hown"):
            assert np.array_equal(a[key], b[key]), key
        assert a["stats"] == b["stats"]
    finally:
        for e in engs:
            e.close()


@pytest.mark.parametrize("seed", range(6))
def test_lru_release_random(seed):
    """Released entries' slots become free: exact LRU takes freed GPU slots first
    (ascending), and a slot appended after its release counts as never stamped."""
    from tracegen import release_plan
    wl = tiny_workload(seed, steps=10)
    tr = Trace(wl)
    sels = padded_selections(tr, 0, seed)
    run_lru_parity(wl, selections=sels, max_append=7, releases=release_plan(tr, sels, seed, frac=0.4))
