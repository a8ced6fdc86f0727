"""Exact LRU over one GPU pool plus one host pool, by brute force (oracle; tests only).

Source: UlaCache summary (paper-daily.com, "UlaCache: Unified Logical
Addressing for Sparse LLM Serving"), section 3: the textbook LRU it compares against stamps every slot with
its last use and looks at every slot of the pool when it picks victims; section 4
reports that PB-LRU's GPU hit rate on replayed traces stays within 0.1
percentage point of exact LRU.

This is a deliberately naive pure-Python implementation (lists, dicts, a full
scan and a sort per step) used only on tiny traces, as an independent
reference for the PB-LRU oracle. Everything except the replacement decision
follows the same readings as the PB-LRU oracle (first-occurrence
de-duplication, hits and misses per unique entry, i-th miss takes the i-th
victim, the victim's rows go to the host slot the miss vacated, appends take
the lowest free GPU slot else the lowest free host slot). The replacement
decision is the textbook one:

* an entry appended into GPU slot s gets stamp ``s - P`` (older than any step,
  ordered by slot, so the initial residents' slot order is their age order);
* a hit or a load at step t sets the slot's stamp to t;
* victims are the free slots in ascending order, then the occupied slots in
  (stamp ascending, slot ascending) order, excluding slots stamped t.

With placement "ring" an append is an access of the last step's round instead:
each appended entry in turn takes the first slot of the victim order of that
round t (free slots ascending, then occupied slots by (stamp, slot), never one
stamped t), is stamped t, and the entry it displaces moves to the lowest free
host slot; with no such slot left it takes the lowest free host slot itself.
"""

from __future__ import annotations

import heapq
from typing import List


class ExactLRUGroup:
    def __init__(self, N: int, P: int, H: int, placement: str = "lowest"):
        assert placement in ("lowest", "ring")
        self.placement = placement
        self.N, self.P, self.H = N, P, H
        self.where = {}                 # la -> ("gpu", slot) | ("host", slot)
        self.gown: List[int] = [-1] * P
        self.hown: List[int] = [-1] * H
        self.stamp: List[int] = [0] * P
        self.t = 0
        self.last = None                # (unique, hits, misses, evictions, from_free, invalid)
        self.last_victims: List[int] = []
        # lowest-first free lists (a heap pops its smallest element)
        self.free_gpu = list(range(P))
        self.free_host = list(range(H))

    def append(self, las) -> None:
        if self.placement == "ring":
            self._append_ring(las)
            return
        for la in [int(x) for x in las]:
            assert la not in self.where
            if self.free_gpu:
                s = heapq.heappop(self.free_gpu)
                self.gown[s] = la
                self.stamp[s] = s - self.P
                self.where[la] = ("gpu", s)
            else:
                h = heapq.heappop(self.free_host)
                self.hown[h] = la
                self.where[la] = ("host", h)

    def _append_ring(self, las) -> None:
        t = self.t
        for la in [int(x) for x in las]:
            assert la not in self.where
            free = sorted(self.free_gpu)
            occupied = [s for s in range(self.P) if self.gown[s] != -1 and self.stamp[s] != t]
            occupied.sort(key=lambda s: (self.stamp[s], s))
            order = free + occupied
            if not order:
                h = heapq.heappop(self.free_host)
                self.hown[h] = la
                self.where[la] = ("host", h)
                continue
            v = order[0]
            old = self.gown[v]
            if old == -1:
                self.free_gpu.remove(v)
                heapq.heapify(self.free_gpu)
            else:
                h = heapq.heappop(self.free_host)
                self.hown[h] = old
                self.where[old] = ("host", h)
            self.gown[v] = la
            self.stamp[v] = t
            self.where[la] = ("gpu", v)

    def release(self, las) -> None:
        """The released entries' slots become free (GPU: back on the free list,
        stamp cleared; host: back on the free list); the addresses become absent."""
        for la in [int(x) for x in las]:
            kind, s = self.where.pop(la)
            if kind == "gpu":
                self.gown[s] = -1
                self.stamp[s] = 0
                heapq.heappush(self.free_gpu, s)
            else:
                self.hown[s] = -1
                heapq.heappush(self.free_host, s)

    def step(self, sel) -> None:
        self.t += 1
        t = self.t
        U, seen, invalid = [], set(), 0
        for row in sel:
            for x in row:
                x = int(x)
                if x == -1:
                    invalid += 1
                elif x not in seen:
                    seen.add(x)
                    U.append(x)
        assert len(U) <= self.P
        hits = [self.where[x][1] for x in U if self.where[x][0] == "gpu"]
        misses = [x for x in U if self.where[x][0] == "host"]
        for s in hits:
            self.stamp[s] = t
        free = sorted(self.free_gpu)
        occupied = [s for s in range(self.P) if self.gown[s] != -1 and self.stamp[s] != t]
        occupied.sort(key=lambda s: (self.stamp[s], s))
        victims = (free + occupied)[: len(misses)]
        evictions = 0
        for la, v in zip(misses, victims):
            h = self.where[la][1]
            old = self.gown[v]
            self.where[la] = ("gpu", v)
            self.gown[v] = la
            self.stamp[v] = t
            if old != -1:
                self.where[old] = ("host", h)
                self.hown[h] = old
                evictions += 1
            else:
                self.free_gpu.remove(v)
                heapq.heapify(self.free_gpu)
                self.hown[h] = -1
                heapq.heappush(self.free_host, h)
        self.last = (len(U), len(hits), len(misses), evictions, len(misses) - evictions, invalid)
        self.last_victims = victims

    def map_array(self):
        """The mapping table in the engine's encoding (list of ints, length N)."""
        out = [0xFFFFFFFF] * self.N
        for la, (kind, s) in self.where.items():
            out[la] = s if kind == "gpu" else (0x80000000 | s)
        return out
