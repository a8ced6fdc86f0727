"""Parity of the engine's second placement of appended entries (ULA_PLACE_RING).

Under this placement an appended entry joins the current bucket on the GPU in
the slot the step's victim order gives next (free, cold, ring oldest to newest,
never the current bucket), the entry displaced from it moves to the lowest free
host slot, and entries left over once no victim remains take free host slots
(UlaCache summary, section 2: the library places new KV; section 3: entries of
the current round stay on the GPU). The oracle's PBLRUGroup(placement="ring")
is pinned on the CPU by a hand-worked example and by the long-ring equivalence
with the brute-force exact LRU; here the engine must match it bit for bit
(mapping table, owners, buckets, statistics, every gathered byte, stored rows)
through every append path: the one-workgroup append (and its place inside a
step's first launch, ula_append_step), the plan / extract / place kernels of a
larger append, and chunked initial loads.
"""

import dataclasses

import numpy as np
import pytest

from gpu_harness import run_parity
from synth import Trace, preset, scaled
from tracegen import padded_selections, release_plan, tiny_workload

pytestmark = pytest.mark.gpu


def _evicting(seed, **kw):
    """A random tiny workload whose appends evict (one to three per request and step)."""
    wl = tiny_workload(seed, **kw)
    return dataclasses.replace(wl, appends=1 + seed % 3, name=f"ring{seed}")


@pytest.mark.parametrize("seed", range(12))
def test_ring_placement_random(seed):
    """Separate ula_append and ula_step calls; the initial load runs in chunks of
    seven entries through the plan / extract / place kernels, the appends of a
    step through the one-workgroup path."""
    wl = _evicting(seed)
    tr = Trace(wl)
    run_parity(wl, selections={0: padded_selections(tr, 0, seed)}, max_append=7, placement=1)


@pytest.mark.parametrize("seed", range(8))
def test_ring_placement_append_step(seed):
    """The step's appends in its first launch (ula_append_step), with the current
    bucket of the step before."""
    wl = _evicting(seed + 40)
    tr = Trace(wl)
    run_parity(wl, selections={0: padded_selections(tr, 0, seed)}, max_append=64, combined=True,
               placement=1, gather_mode="split" if wl.layers > 1 else "layer")


@pytest.mark.parametrize("ring", [1, 2, 9])
def test_ring_placement_ring_lengths(ring):
    wl = dataclasses.replace(preset("tiny_4x4k"), ring=ring, name=f"tiny_ring{ring}_place")
    run_parity(wl, placement=1, combined=ring != 2)


@pytest.mark.parametrize("name,factor,steps,combined", [
    ("r16_64k_g1x3", 16, 8, True),
    ("spec3_r128_64k128k_g4", 32, 5, True),     # 384 appends per step: the bulk append kernels
    ("evict_r256_128k_g2", 32, 6, False),
])
def test_ring_placement_scaled(name, factor, steps, combined):
    wl = scaled(preset(name), factor)
    run_parity(wl, steps=steps, max_append=1 << 15, check_every=1, combined=combined, placement=1,
               gather_mode="split" if wl.layers > 1 else "layer")


@pytest.mark.parametrize("appends,pool_frac", [(1, 0.5), (2, 0.0)])
def test_ring_placement_many_appends(appends, pool_frac):
    """300 and 600 appends per step (more than one workgroup takes), with room on
    the GPU and with a full GPU pool; chunks of 256 through the bulk kernels."""
    from synth.configs import Workload
    wl = Workload(name=f"ring_many{appends}", requests=300, ctx_fixed=2048, ctx_range=None,
                  sets_per_request=1, draft_keep=0.0, groups=1, layers=2, k=64, pool_frac=pool_frac,
                  pool_slots=None if pool_frac else 40_000, ring=4, steps=4, appends=appends, overlap=0.8,
                  p_recent=0.7, window=256, row_bytes=64, seed=3)
    run_parity(wl, max_append=256, combined=True, placement=1)


@pytest.mark.parametrize("seed", range(4))
def test_ring_placement_with_releases(seed):
    """Releases between steps free GPU slots, which the next appends take first."""
    wl = _evicting(seed + 80, steps=10)
    tr = Trace(wl)
    sels = padded_selections(tr, 0, seed)
    ora = run_parity(wl, selections={0: sels}, max_append=7, check_every=1, placement=1,
                     releases=release_plan(tr, sels, seed, frac=0.4))
    assert ora[0].flag == tr.steps


def test_ring_placement_refused_with_exact_lru():
    from serving_pb_lru_amd import Engine, UlaError
    tr = Trace(preset("tiny_4x4k"))
    wl = tr.wl
    with pytest.raises(UlaError) as e:
        Engine(1, wl.layers, wl.row_bytes, wl.ring, tr.N, tr.P, tr.H, tr.n_sets, tr.k, policy=1, placement=1)
    assert e.value.name == "EINVAL"
