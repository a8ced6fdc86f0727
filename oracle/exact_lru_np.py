"""Exact LRU over one GPU pool plus one host pool, with numpy arrays (oracle; tests only).

The same textbook policy as ``exact_lru.ExactLRUGroup`` (UlaCache summary,
paper-daily.com, section 3: one timestamp per slot, a scan of the whole pool for
the victims; section 4 compares PB-LRU against it), written with arrays so that
it runs at the workloads' full sizes. Each step follows the definition in order:

1. step number t = previous + 1;
2. distinct valid addresses U in first-occurrence row-major order (-1 is
   padding), each looked up: hits (on the GPU) and misses (in the host pool);
   more distinct addresses than GPU slots is the capacity error, nothing changes;
3. every hit slot is stamped t;
4. victims = the free GPU slots in ascending order, then the occupied slots
   not stamped t, by (stamp, slot) ascending (one library sort); the i-th miss
   takes the i-th victim;
5. the missed entry moves to its victim slot, which is stamped t; the victim's
   entry moves to the host slot the miss vacated, or that host slot becomes
   free when the victim slot was free.

Appends take the lowest free GPU slot (stamped s - P: older than any step and
ordered by slot), else the lowest free host slot, in list order. Metadata only:
the rows of an entry are a closed form of its address, so gathers and stored
rows are checked against that form. Pinned against the brute-force
``ExactLRUGroup`` on random traces (tests/test_oracle_vs_lru.py).
"""

from __future__ import annotations

import numpy as np

ABSENT = 0xFFFFFFFF
HOST = 0x80000000


class CapacityError(Exception):
    pass


class ExactLRUArrays:
    def __init__(self, N: int, P: int, H: int, B: int):
        self.N, self.P, self.H, self.B = N, P, H, B
        self.map = np.full(N, ABSENT, dtype=np.uint32)
        self.gown = np.full(P, -1, dtype=np.int32)
        self.hown = np.full(H, -1, dtype=np.int32)
        self.stamp = np.zeros(P, dtype=np.int64)
        self.free_gpu = np.ones(P, dtype=bool)
        self.free_host = np.ones(H, dtype=bool)
        self.t = 0
        self.last = (0, 0, 0, 0, 0, 0)
        self.last_victims = np.zeros(0, dtype=np.int64)

    def append(self, las) -> None:
        las = np.asarray(las, dtype=np.int64).reshape(-1)
        if las.size == 0:
            return
        assert np.all(self.map[las] == ABSENT) and np.unique(las).size == las.size
        gslots = np.flatnonzero(self.free_gpu)[: las.size]          # lowest free GPU slots, in order
        ng = gslots.size
        hslots = np.flatnonzero(self.free_host)[: las.size - ng]     # then the lowest free host slots
        assert ng + hslots.size == las.size, "no room for the append"
        g_las, h_las = las[:ng], las[ng:]
        self.map[g_las] = gslots.astype(np.uint32)
        self.gown[gslots] = g_las
        self.stamp[gslots] = gslots - self.P
        self.free_gpu[gslots] = False
        self.map[h_las] = (HOST | hslots).astype(np.uint32)
        self.hown[hslots] = h_las
        self.free_host[hslots] = False

    def release(self, las) -> None:
        """The released entries' slots become free; the addresses become absent."""
        las = np.asarray(las, dtype=np.int64).reshape(-1)
        if las.size == 0:
            return
        assert np.unique(las).size == las.size and np.all(self.map[las] != ABSENT)
        loc = self.map[las].astype(np.int64)
        on_gpu = (loc & HOST) == 0
        s = loc[on_gpu]
        self.gown[s] = -1
        self.stamp[s] = 0
        self.free_gpu[s] = True
        h = loc[~on_gpu] & ~HOST
        self.hown[h] = -1
        self.free_host[h] = True
        self.map[las] = ABSENT

    def step(self, sel) -> None:
        flat = np.asarray(sel, dtype=np.int64).reshape(-1)
        valid = flat != -1
        invalid = int(flat.size - valid.sum())
        vals = flat[valid]
        assert np.all((vals >= 0) & (vals < self.N)) and np.all(self.map[vals] != ABSENT)
        uniq, first = np.unique(vals, return_index=True)
        U = uniq[np.argsort(first, kind="stable")]                   # first-occurrence order
        if U.size > self.P:
            raise CapacityError
        t = self.t + 1
        loc = self.map[U].astype(np.int64)
        on_gpu = (loc & HOST) == 0
        hits = loc[on_gpu]
        misses = U[~on_gpu]
        mh = loc[~on_gpu] & ~HOST
        self.stamp[hits] = t
        free = np.flatnonzero(self.free_gpu)
        occ = np.flatnonzero(~self.free_gpu & (self.stamp != t))
        occ = occ[np.lexsort((occ, self.stamp[occ]))]               # by (stamp, slot)
        victims = np.concatenate([free, occ])[: misses.size]
        assert victims.size == misses.size
        old = self.gown[victims].copy()
        self.map[misses] = victims.astype(np.uint32)
        self.gown[victims] = misses
        self.stamp[victims] = t
        self.free_gpu[victims] = False
        ev = old != -1
        self.map[old[ev]] = (HOST | mh[ev]).astype(np.uint32)
        self.hown[mh[ev]] = old[ev]
        self.hown[mh[~ev]] = -1
        self.free_host[mh[~ev]] = True
        self.t = t
        nev = int(ev.sum())
        self.last = (int(U.size), int(hits.size), int(misses.size), nev, int(misses.size) - nev, invalid)
        self.last_victims = victims

    def export_state(self) -> dict:
        """The engine's exported form: only the free set among the bitsets."""
        W = (self.P + 31) // 32
        bits = np.zeros((self.B + 2, W * 32), dtype=bool)
        bits[0, : self.P] = self.free_gpu
        words = np.packbits(bits.reshape(self.B + 2, W, 32)[:, :, ::-1], axis=2, bitorder="big")
        words = words.view(">u4").reshape(self.B + 2, W).astype(np.uint32)
        stamps = np.where(self.free_gpu, 0, self.stamp).astype(np.int32)
        return dict(map=self.map.copy(), gown=self.gown.copy(), hown=self.hown.copy(), bitsets=words,
                    cur=self.t % self.B, flag=self.t, stats=self.last, stamps=stamps)
