"""Full-size parity on the GPU: every workload preset at its real sizes.

The PB-LRU cases drive the engine as bench.py does (each step's appends and
the step in one ula_append_step call; layer 0 gathered alone, the later layers
of the group in one ula_gather_layers launch); the exact-LRU cases use the
separate calls (ula_append, ula_step, one ula_gather per layer).

After the initial load and after every step, the digest of the engine's
exported state (mapping table, owners, bucket bitsets, completion counter, step
statistics) must equal the digest the CPU oracle produced for the same seeded
inputs (tests/golden/digests_<workload>.json, written by
tests/golden/make_state_digests.py from oracle/ alone), and so must the step
statistics ula_sync returns. The current bucket in the digest is derived from
the counter on both sides (the ring advances once per step); which bucket the
step's entries went to is in the bitsets. Every gathered byte of every layer
is compared after every step with its closed form (row contents are a function
of group, address and layer, generated on the device by synth's HIP generator,
itself pinned to the numpy one), zeros for padding. Exporting leaves the staged
evicted rows staged, so every step's write-back still happens inside the next
step; the stored rows of sampled addresses (wherever they live, GPU or host
pool) are read back every eighth step and after the last, which writes the
staged rows out first.

The second placement of appended entries (into the current bucket, evicting)
is checked the same way against the oracle's placement "ring"
(tests/golden/digests_ring_<workload>.json).

The exact-LRU policy is checked the same way against the array form of the
oracle's exact LRU (tests/golden/digests_lru_<workload>.json, timestamps
included), on every workload and on three of the 24 groups of the largest.

Layer groups are independent (their own pools, maps and buckets), so each
group runs in an engine of its own; that keeps the pinned host pool of the
24-group workload within one group's share at a time.
"""

import json
import os

import numpy as np
import pytest

from digests import digest
from gpu_harness import gather_layers_by, say
from synth import Trace, preset, rows_for

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _golden(name, policy=0, placement=0):
    fname = f"digests_lru_{name}.json" if policy else (
        f"digests_ring_{name}.json" if placement else f"digests_{name}.json")
    with open(os.path.join(HERE, "golden", fname)) as f:
        return json.load(f)


def _cmp(got, want, where):
    for k in ("map", "gown", "hown", "bitsets", "cur", "flag", "stats", "stamps"):
        if k in want:
            assert got[k] == want[k], f"{where}: {k} differs (engine {got[k]}, oracle {want[k]})"


def run_group(name: str, g: int, samples: int = 128, policy: int = 0, bench_calls: bool = True,
              placement: int = 0):
    import torch
    from serving_pb_lru_amd import Engine
    from synth.device import rows_device

    wl = preset(name)
    tr = Trace(wl)
    gold = _golden(name, policy, placement)["groups"][g]
    say(f"full parity {name} group {g} policy {policy} placement {placement}: N={tr.N} P={tr.P} "
        f"H={tr.H} steps={tr.steps}")
    eng = Engine(1, wl.layers, wl.row_bytes, wl.ring, tr.N, tr.P, tr.H, tr.n_sets, tr.k,
                 max_append=1 << 16, policy=policy, placement=placement)
    rows = lambda las: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    rng = np.random.default_rng([g, 2024])
    try:
        order = tr.initial_load_order()
        for s in range(0, order.size, 1 << 18):
            las = order[s:s + (1 << 18)]
            eng.append(0, las, rows(las))
        _cmp(digest(eng.export_state(0)), gold[0], f"{name} g{g} after load")
        known = [order]
        sels = tr.selections(g)
        for t in range(1, tr.steps + 1):
            sel = next(sels)
            dsel = torch.from_numpy(sel).cuda()
            app = tr.appends(t)
            known.append(app)
            if bench_calls:
                eng.append_step(0, app, rows(app), dsel)
                outs = gather_layers_by(eng, 0, wl.layers, dsel, "split")
            else:
                if app.size:
                    eng.append(0, app, rows(app))
                eng.step(0, dsel)
                outs = gather_layers_by(eng, 0, wl.layers, dsel, "layer")
            stats = eng.sync()[0]
            assert list(stats) == gold[t]["stats"], f"{name} g{g} step {t}: ula_sync stats {stats}"
            _cmp(digest(eng.export_state(0)), gold[t], f"{name} g{g} step {t}")
            # every gathered byte against its closed form, on the device
            flat = dsel.reshape(-1)
            want = rows(sel.reshape(-1))
            want[flat == -1] = 0
            for l in range(wl.layers):
                got = outs[l].reshape(-1, wl.row_bytes)
                if not torch.equal(got, want[:, l]):
                    bad = (got != want[:, l]).any(dim=1).nonzero().reshape(-1)[:5].tolist()
                    raise AssertionError(f"{name} g{g} step {t} layer {l}: gathered rows differ, "
                                         f"first rows {bad}")
            del want
            if t % 8 == 0 or t == tr.steps:
                pool = np.concatenate(known)
                probe = pool[rng.choice(pool.size, size=samples, replace=False)]
                assert np.array_equal(eng.read_rows(0, probe),
                                      rows_for(wl.seed, g, probe, wl.layers, wl.row_bytes)), \
                    f"{name} g{g} step {t}: stored rows differ"
    finally:
        eng.close()


CASES = ([("tiny_4x4k", 0), ("r16_64k_g1x3", 0)]
         + [("r64_64k128k_g24x3", g) for g in range(24)]
         + [("spec3_r128_64k128k_g4", g) for g in range(4)]
         + [("evict_r256_128k_g2", g) for g in range(2)]
         + [("evict_r256_128k_g2_ctl98", g) for g in range(2)])


@pytest.mark.parametrize("name,g", CASES, ids=[f"{n}-g{g}" for n, g in CASES])
def test_full_size_parity(name, g):
    run_group(name, g)


# exact LRU against the array form of the oracle's exact LRU (digests with timestamps)
LRU_CASES = ([("tiny_4x4k", 0), ("r16_64k_g1x3", 0)]
             + [("r64_64k128k_g24x3", g) for g in (0, 11, 23)]
             + [("spec3_r128_64k128k_g4", g) for g in range(4)]
             + [("evict_r256_128k_g2", g) for g in range(2)]
             + [("evict_r256_128k_g2_ctl98", g) for g in range(2)])


@pytest.mark.parametrize("name,g", LRU_CASES, ids=[f"lru-{n}-g{g}" for n, g in LRU_CASES])
def test_full_size_lru_parity(name, g):
    run_group(name, g, policy=1, bench_calls=False)


# appends placed in the current bucket (ULA_PLACE_RING) against the oracle's
# placement "ring" (tests/golden/digests_ring_<workload>.json)
RING_CASES = ([("tiny_4x4k", 0), ("r16_64k_g1x3", 0)]
              + [("r64_64k128k_g24x3", g) for g in (0, 23)]
              + [("spec3_r128_64k128k_g4", g) for g in range(4)]
              + [("evict_r256_128k_g2", g) for g in range(2)]
              + [("evict_r256_128k_g2_ctl98", g) for g in range(2)])


@pytest.mark.parametrize("name,g", RING_CASES, ids=[f"ring-{n}-g{g}" for n, g in RING_CASES])
def test_full_size_ring_placement_parity(name, g):
    run_group(name, g, placement=1)
