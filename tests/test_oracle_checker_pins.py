"""Pins of the oracle's checkers: each one must fail on the state it rules out.

oracle/invariants.py states I1-I6 and I9 (UlaCache summary, section 2: an entry
lives in exactly one pool in DP mode; section 3: buckets, the current bucket is
never a victim, data moves before the mapping changes). These tests take a
valid state, corrupt one property at a time and expect the checker to raise,
so a checker that went lax would show here. The same is done for the two
bitset packers (pblru.pack_bits and the exact-LRU export) against a brute-force
bit loop, and for the victim-order invariants against planted mistakes in the
oracle (tests/oracle_mutants.py).
"""

import copy

import numpy as np
import pytest

from oracle.exact_lru_np import ExactLRUArrays
from oracle.invariants import check_state, check_step
from oracle.pblru import HOST_BIT, PBLRUGroup, pack_bits
from oracle_mutants import ColdBeforeFree, CurrentBucketEvictable

# a pool whose size is not a multiple of 32, so the last bitset word has spare bits
N, P, H, B = 100, 45, 55, 3


def _scenario(cls=PBLRUGroup):
    """A group with free GPU slots before a step whose misses exceed them:
    load 70 entries (45 on the GPU, 25 on the host), release 5 GPU entries, then
    select 3 GPU entries (hits) and 8 host entries (misses)."""
    g = cls(N, P, H, B, 1, 16, full_data=False)
    g.append(np.arange(70), None)
    g.step(np.array([[0, 1, 2, 3]]))          # something in the ring before the real step
    g.release(np.array([10, 11, 12, 13, 14]))
    prev = g.export_state()
    sel = np.array([[5, 6, 7, 50, 51, 52, 53], [54, 55, 56, 57, 5, -1, 50]])
    g.step(sel)
    U, hits, _, _, victims = g.last_lists
    return prev, g.export_state(), U, hits, victims


def _bits(words):
    b = np.unpackbits(np.asarray(words, dtype="<u4").view(np.uint8), bitorder="little")
    return b.astype(bool)


def _set_bit(words, s, on=True):
    w = words.copy()
    if on:
        w[s >> 5] |= np.uint32(1 << (s & 31))
    else:
        w[s >> 5] &= np.uint32(~(1 << (s & 31)) & 0xFFFFFFFF)
    return w


def test_scenario_is_valid():
    prev, st, U, hits, victims = _scenario()
    check_state(prev, P, H)
    check_step(prev, st, P, H, U=U, victims=victims, hit_slots=hits)
    unique, nh, nm, ev, ff, inv = st["stats"]
    assert (nh, nm, ff, ev) == (3, 8, 5, 3) and inv == 1   # the step uses free slots, then evicts


def _occupied_gpu(st):
    return np.flatnonzero(np.asarray(st["gown"]) != -1)


def _corruptions(st, U, hits):
    """(name, corrupted state, expected message pattern) for check_state."""
    out = []
    gown, hown, m = st["gown"], st["hown"], st["map"]
    occ = _occupied_gpu(st)
    s1, s2 = int(occ[0]), int(occ[1])
    free_h = int(np.flatnonzero(hown == -1)[0])

    c = copy.deepcopy(st)                              # an entry held in both pools
    c["hown"][free_h] = gown[s1]
    out.append(("both pools", c, "host owner -> map|held twice"))

    c = copy.deepcopy(st)                              # owners swapped, map unchanged
    c["gown"][s1], c["gown"][s2] = gown[s2], gown[s1]
    out.append(("owner swap", c, "owner mismatch|owner -> map"))

    la_h = int(np.flatnonzero((m != 0xFFFFFFFF) & ((m & HOST_BIT) != 0))[0])
    c = copy.deepcopy(st)                              # map names another host slot
    c["map"][la_h] = HOST_BIT | np.uint32(free_h)
    out.append(("map to wrong host slot", c, "host slot owner mismatch"))

    c = copy.deepcopy(st)                              # appended, but held by no slot
    c["hown"][int(m[la_h] & ~HOST_BIT)] = -1
    out.append(("held nowhere", c, "mismatch|held nowhere"))

    cur = 2 + st["cur"]
    s_cur = int(np.flatnonzero(_bits(st["bitsets"][cur])[:P])[0])
    c = copy.deepcopy(st)                              # two buckets share a slot
    c["bitsets"][1] = _set_bit(c["bitsets"][1], s_cur)
    out.append(("shared slot", c, "partition"))

    c = copy.deepcopy(st)                              # a slot in no bucket
    c["bitsets"][cur] = _set_bit(c["bitsets"][cur], s_cur, on=False)
    out.append(("slot in no bucket", c, "partition"))

    c = copy.deepcopy(st)                              # a bit at or beyond P
    c["bitsets"][1] = _set_bit(c["bitsets"][1], P)
    out.append(("bit beyond the pool", c, "beyond the pool"))

    c = copy.deepcopy(st)                              # an occupied slot labelled free
    c["bitsets"][cur] = _set_bit(c["bitsets"][cur], s_cur, on=False)
    c["bitsets"][0] = _set_bit(c["bitsets"][0], s_cur)
    out.append(("occupied slot in free", c, "free bucket differs"))
    return out


@pytest.mark.parametrize("i", range(8))
def test_check_state_rejects_each_corruption(i):
    prev, st, U, hits, victims = _scenario()
    name, bad, pattern = _corruptions(st, U, hits)[i]
    with pytest.raises(AssertionError, match=pattern):
        check_state(bad, P, H)


def _step_corruptions(prev, st, U, hits, victims):
    out = []
    c = copy.deepcopy(st)
    c["flag"] += 1
    out.append(("flag != step", c, {}, "I9"))
    c = copy.deepcopy(st)
    c["cur"] = prev["cur"]
    out.append(("ring not advanced", c, {}, "advance"))
    u, h, mi, ev, ff, inv = st["stats"]
    c = copy.deepcopy(st)
    c["stats"] = (u, h + 1, mi, ev, ff, inv)
    out.append(("hits + misses != unique", c, {}, "hits \\+ misses"))
    c = copy.deepcopy(st)
    c["stats"] = (u, h, mi, ev + 1, ff, inv)
    out.append(("evictions do not add up", c, {}, "from_free \\+ evictions"))
    c = copy.deepcopy(st)
    c["stats"] = (u, h, mi, ev - 1, ff + 1, inv)
    out.append(("occupancy growth", c, {}, "grow by from_free"))
    # ring[cur] != U: one unique entry's slot relabelled cold (partition kept)
    cur = 2 + st["cur"]
    s_cur = int(np.flatnonzero(_bits(st["bitsets"][cur])[:P])[0])
    c = copy.deepcopy(st)
    c["bitsets"][cur] = _set_bit(c["bitsets"][cur], s_cur, on=False)
    c["bitsets"][1] = _set_bit(c["bitsets"][1], s_cur)
    out.append(("current bucket != U", c, {}, "I3"))
    # a selected entry left on the host (swap it with a host-resident entry)
    c = copy.deepcopy(st)
    la_u = int(U[0])
    la_h = int(np.flatnonzero((c["map"] != 0xFFFFFFFF) & ((c["map"] & HOST_BIT) != 0))[0])
    s, h = int(c["map"][la_u]), int(c["map"][la_h] & ~HOST_BIT)
    c["map"][la_u], c["map"][la_h] = HOST_BIT | np.uint32(h), np.uint32(s)
    c["gown"][s], c["hown"][h] = la_h, la_u
    out.append(("selected entry on the host", c, {"U": U}, "not GPU-resident"))
    # a victim among the hits
    out.append(("victim among the hits", copy.deepcopy(st),
                {"victims": np.concatenate([victims, hits[:1]]), "hit_slots": hits}, "I4"))
    return out


@pytest.mark.parametrize("i", range(8))
def test_check_step_rejects_each_corruption(i):
    prev, st, U, hits, victims = _scenario()
    name, bad, kw, pattern = _step_corruptions(prev, st, U, hits, victims)[i]
    with pytest.raises(AssertionError, match=pattern):
        check_step(prev, bad, P, H, **kw)


def test_eviction_before_the_pool_is_full_is_caught():
    """I5 (eviction only once the GPU pool is full) on an oracle that takes cold
    slots before free ones."""
    prev, st, U, hits, victims = _scenario(ColdBeforeFree)
    with pytest.raises(AssertionError, match="I5"):
        check_step(prev, st, P, H, U=U, victims=victims, hit_slots=hits)


def test_current_bucket_victim_is_caught():
    """I3/I4 on an oracle that may evict from the current bucket: with most slots
    in an older ring bucket, a step with more misses than cold slots takes this
    step's hits."""
    g = CurrentBucketEvictable(N, P, H, B, 1, 16, full_data=False)
    g.append(np.arange(70), None)
    g.step(np.arange(40)[None, :])                 # slots 0..39 into ring[1], 5 left in cold
    prev = g.export_state()
    sel = np.array([list(range(0, 10)) + list(range(50, 60))])   # 10 hits, 10 misses
    g.step(sel)
    U, hits, _, _, victims = g.last_lists
    with pytest.raises(AssertionError, match="I3|I4"):
        check_step(prev, g.export_state(), P, H, U=U, victims=victims, hit_slots=hits)


# ---- bitset packing, against a plain bit loop ------------------------------
def _pack_brute(mask):
    words = [0] * ((len(mask) + 31) // 32)
    for s, on in enumerate(mask):
        if on:
            words[s >> 5] |= 1 << (s & 31)
    return words


@pytest.mark.parametrize("size", [1, 31, 32, 33, 45, 64, 100, 257])
def test_pack_bits_matches_a_bit_loop(size):
    rng = np.random.default_rng(size)
    for _ in range(5):
        mask = rng.random(size) < rng.random()
        assert pack_bits(mask).tolist() == _pack_brute(mask.tolist())


@pytest.mark.parametrize("seed", range(6))
def test_exact_lru_export_bitsets_match_a_bit_loop(seed):
    """ExactLRUArrays.export_state packs the free set with a reversed-bit big-endian
    trick; it must equal the plain layout (slot s = bit s & 31 of word s >> 5),
    other buckets empty."""
    rng = np.random.default_rng([seed, 5])
    n, p, h = 200, int(rng.integers(20, 90)), 150
    g = ExactLRUArrays(n, p, h, 4)
    g.append(rng.permutation(n)[:int(rng.integers(p // 2, n))])
    for t in range(4):
        appended = np.flatnonzero(g.map != 0xFFFFFFFF)
        g.step(rng.choice(appended, size=min(appended.size, p // 2), replace=False))
        alive = np.flatnonzero(g.map != 0xFFFFFFFF)
        g.release(rng.choice(alive, size=int(rng.integers(0, 5)), replace=False))
        st = g.export_state()
        assert st["bitsets"].shape == (6, (p + 31) // 32)
        assert st["bitsets"][0].tolist() == _pack_brute(g.free_gpu.tolist())
        assert not st["bitsets"][1:].any()
