"""Structural invariants of the residency state (oracle; tests only).

Each check is stated from the UlaCache summary (paper-daily.com, "UlaCache:
Unified Logical Addressing for Sparse LLM Serving") or from the readings that
the oracle states. They apply to any exported state, the oracle's or the
engine's, given as a dict with ``map``, ``gown``, ``hown``, ``bitsets``
([free, cold, ring...] as uint32 words), ``cur``, ``flag`` and ``stats``
(unique, hits, misses, evictions, from_free, invalid).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

ABSENT = 0xFFFFFFFF
HOST_BIT = 0x80000000


def unpack(words: np.ndarray, P: int) -> np.ndarray:
    """uint32 words -> bool [P] (slot s = bit s & 31 of word s >> 5)."""
    b = np.unpackbits(np.asarray(words, dtype="<u4").view(np.uint8), bitorder="little")
    return b[:P].astype(bool), b[P:]


def check_state(st: dict, P: int, H: int) -> None:
    """I1 exclusivity (section 2, DP mode) and I2 bucket partition (section 3)."""
    m = np.asarray(st["map"], dtype=np.uint32).astype(np.int64)
    gown = np.asarray(st["gown"], dtype=np.int64)
    hown = np.asarray(st["hown"], dtype=np.int64)
    assert gown.size == P and hown.size == H, "owner arrays of the wrong size"

    # I1: an entry is on the GPU or on the host, never both, and the mapping
    # table and the owners agree both ways
    appended = m != ABSENT
    on_host = appended & ((m & HOST_BIT) != 0)
    on_gpu = appended & ~on_host
    la_g = np.flatnonzero(on_gpu)
    la_h = np.flatnonzero(on_host)
    assert (gown[m[la_g]] == la_g).all(), "map -> GPU slot owner mismatch"
    assert (hown[m[la_h] & ~HOST_BIT] == la_h).all(), "map -> host slot owner mismatch"
    occ_g = np.flatnonzero(gown != -1)
    occ_h = np.flatnonzero(hown != -1)
    assert (m[gown[occ_g]] == occ_g).all(), "GPU owner -> map mismatch"
    assert (m[hown[occ_h]] == (occ_h | HOST_BIT)).all(), "host owner -> map mismatch"
    owners = np.concatenate([gown[occ_g], hown[occ_h]])
    assert np.unique(owners).size == owners.size, "an entry is held twice"
    assert owners.size == int(appended.sum()), "an appended entry is held nowhere"

    # I2: free, cold and the ring buckets partition the GPU slots; free = empty slots
    masks = []
    for w in st["bitsets"]:
        bits, tail = unpack(w, P)
        assert not tail.any(), "bits beyond the pool are set"
        masks.append(bits)
    total = np.sum(masks, axis=0)
    assert (total == 1).all(), "buckets do not partition the GPU slots"
    assert (masks[0] == (gown == -1)).all(), "free bucket differs from the empty slots"


def check_step(prev: dict, st: dict, P: int, H: int, U: Optional[np.ndarray] = None,
               victims: Optional[np.ndarray] = None, hit_slots: Optional[np.ndarray] = None) -> None:
    """I3-I6 and I9 across one step (section 3 and the stated readings)."""
    check_state(st, P, H)
    unique, hits, misses, evictions, from_free, invalid = st["stats"]
    B = len(st["bitsets"]) - 2
    # I9: the completion counter is the step number
    assert st["flag"] == prev["flag"] + 1, "I9: the completion counter is not the step number"
    assert st["cur"] == (prev["cur"] + 1) % B, "the ring did not advance by one bucket"
    # I6: conservation
    assert hits + misses == unique, "I6: hits + misses != unique"
    assert from_free + evictions == misses, "I6: from_free + evictions != misses"
    occ_prev = int((np.asarray(prev["gown"]) != -1).sum())
    occ_now = int((np.asarray(st["gown"]) != -1).sum())
    assert occ_now - occ_prev == from_free, "I6: occupied GPU slots did not grow by from_free"
    # I5: eviction starts only once the pool is full
    free_prev = P - occ_prev
    assert from_free == min(misses, free_prev), \
        f"I5: eviction while free slots remained (from_free {from_free}, misses {misses}, free {free_prev})"
    # I3: the current bucket holds exactly this step's unique entries, all on the GPU
    cur_bits, _ = unpack(st["bitsets"][2 + st["cur"]], P)
    assert int(cur_bits.sum()) == unique, "I3: the current bucket does not hold exactly the unique entries"
    if U is not None:
        m = np.asarray(st["map"], dtype=np.int64)[np.asarray(U, dtype=np.int64)]
        assert ((m & HOST_BIT) == 0).all(), "a selected entry is not GPU-resident"
        assert cur_bits[m].all() and np.unique(m).size == unique, \
            "I3: a selected entry is outside the current bucket"
    # I4: no victim was taken from the current bucket
    if victims is not None and hit_slots is not None:
        assert np.intersect1d(victims, hit_slots).size == 0, "I4: a victim was taken from the current bucket"
