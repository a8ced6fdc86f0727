"""PB-LRU replacement state of one layer group (oracle; test infrastructure only).

Source: UlaCache summary (paper-daily.com, "UlaCache: Unified Logical
Addressing for Sparse LLM Serving").

* Section 2 (unified logical addresses): an entry's logical address never
  changes; a table maps it to the GPU or host slot that holds it, so moving an
  entry means copying its rows and rewriting one table entry. In the DP form
  there is one GPU pool and one host pool per GPU and each entry is in one of
  them only. A layer group resolves and de-duplicates its shared selection once.
* Section 3 (PB-LRU): the slots touched in one scheduling round share a bucket;
  a group has a ring of such buckets and one cold bucket. Each round moves the
  ring index on; the slots still labelled with the bucket being reused become
  cold, a relabelling only. Victims are taken from free slots, then cold, then
  the other ring buckets by age, never from the running round's bucket. Rows
  move before the table changes, and a completion signal comes last.

Readings where the pages are silent (each restated where it is used):

* a scheduling round is one ``step`` call of one group; the ring advances at
  the start of the step, before hits are marked; ``cur`` starts at 0;
* de-duplication keeps the first occurrence in row-major (set, index) order;
  ``-1`` entries are padding; hits and misses are counted per unique entry;
* inside a bucket victims are taken in ascending slot order; ring buckets are
  visited from ``cur+1`` (oldest) to ``cur-1`` (newest), modulo the ring;
* the i-th miss (in unique order) takes the i-th victim; the victim's rows go
  to the host slot that the miss vacated (a swap), or that host slot becomes
  free when the victim slot was free;
* slots loaded by the step, like hits, join the current bucket;
* an append takes the lowest free GPU slot (joining the cold bucket), else the
  lowest free host slot; appends never evict (placement "lowest", the default);
  the alternative placement "ring" puts each appended entry on the GPU in the
  current bucket, in the slot the next victim of the step's order would be
  (free, cold, ring oldest -> newest, never the current bucket), and sends that
  slot's entry to the lowest free host slot; once no victim is left, entries
  take the lowest free host slots;
* more unique entries than GPU slots is a capacity error and changes nothing;
* the completion signal is a per-group step counter ``flag``.

The canonical state compared with the engine after every step: ``map``
(``s`` = GPU slot s, ``0x80000000 | h`` = host slot h, ``0xFFFFFFFF`` = never
appended), the owners ``gown``/``hown`` (-1 = empty), the bucket bitsets
(free, cold, ring[0..B-1]; slot s is bit ``s & 31`` of word ``s >> 5``),
``cur``, ``flag`` and the step statistics.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

ABSENT = np.uint32(0xFFFFFFFF)
HOST_BIT = np.uint32(0x80000000)


class OracleError(Exception):
    """An error the engine must report with the same name; state is unchanged."""

    def __init__(self, name: str, msg: str = ""):
        super().__init__(f"{name}: {msg}" if msg else name)
        self.name = name


@dataclass
class StepStats:
    unique: int = 0
    hits: int = 0
    misses: int = 0
    evictions: int = 0
    from_free: int = 0
    invalid: int = 0

    def as_tuple(self):
        return (self.unique, self.hits, self.misses, self.evictions, self.from_free, self.invalid)


def pack_bits(mask: np.ndarray) -> np.ndarray:
    """Bool [P] -> uint32 [ceil(P/32)], slot s = bit (s & 31) of word (s >> 5)."""
    P = mask.size
    W = (P + 31) // 32
    b = np.packbits(np.asarray(mask, dtype=bool), bitorder="little")
    b = np.concatenate([b, np.zeros(W * 4 - b.size, dtype=np.uint8)])
    return b.view("<u4").astype(np.uint32)


class PBLRUGroup:
    """The state of one layer group: map, owners, buckets and (optionally) pools."""

    def __init__(self, N: int, P: int, H: int, B: int, layers: int, row_bytes: int,
                 full_data: bool = True, placement: str = "lowest"):
        if B < 1 or P < 1 or H < 0 or N < 1 or layers < 1:
            raise OracleError("EINVAL", "bad sizes")
        if placement not in ("lowest", "ring"):
            raise OracleError("EINVAL", "placement is 'lowest' or 'ring'")
        self.placement = placement
        self.N, self.P, self.H, self.B = N, P, H, B
        self.layers, self.row_bytes = layers, row_bytes
        self.full_data = full_data
        # init: nothing appended, every GPU slot free, no bucket populated
        self.map = np.full(N, ABSENT, dtype=np.uint32)
        self.gown = np.full(P, -1, dtype=np.int32)
        self.hown = np.full(H, -1, dtype=np.int32)
        self.free = np.ones(P, dtype=bool)
        self.cold = np.zeros(P, dtype=bool)
        self.ring = np.zeros((B, P), dtype=bool)
        self.cur = 0
        self.flag = 0
        self.last = StepStats()
        self.last_lists = None     # (U, hit slots, misses, miss host slots, victims) of the last step
        if full_data:
            self.gpu = np.zeros((P, layers, row_bytes), dtype=np.uint8)
            self.host = np.zeros((H, layers, row_bytes), dtype=np.uint8)

    # ------------------------------------------------------------------
    def append(self, las: np.ndarray, rows: Optional[np.ndarray]) -> None:
        """Make new logical entries resident (placement is the library's choice, section 2).

        Reading: in list order, each entry takes the lowest free GPU slot (and
        joins the cold bucket) if one exists, otherwise the lowest free host
        slot; appends never evict. Taking the lowest remaining free slot one
        entry at a time hands out the free slots in ascending order, so the
        first min(n, #free) entries get the free GPU slots in ascending order
        and the rest get the free host slots in ascending order.
        """
        las = np.asarray(las, dtype=np.int64).reshape(-1)
        n = las.size
        if n == 0:
            return
        if las.min() < 0 or las.max() >= self.N:
            raise OracleError("ERANGE", "address out of range")
        if np.unique(las).size != n:
            raise OracleError("EDUP", "address repeated in one append")
        if (self.map[las] != ABSENT).any():
            raise OracleError("EDUP", "address already appended")
        free_gpu = np.flatnonzero(self.free)
        free_host = np.flatnonzero(self.hown == -1)
        if n > free_gpu.size + free_host.size:
            raise OracleError("EHOSTFULL", "no room for the append")
        if self.full_data:
            rows = np.asarray(rows, dtype=np.uint8).reshape(n, self.layers, self.row_bytes)
        if self.placement == "ring":
            self._append_ring(las, rows, free_host)
            return
        n_gpu = min(n, free_gpu.size)
        s = free_gpu[:n_gpu]
        la_g = las[:n_gpu]
        self.map[la_g] = s.astype(np.uint32)
        self.gown[s] = la_g
        self.free[s] = False
        self.cold[s] = True
        h = free_host[: n - n_gpu]
        la_h = las[n_gpu:]
        self.map[la_h] = HOST_BIT | h.astype(np.uint32)
        self.hown[h] = la_h
        if self.full_data:
            self.gpu[s] = rows[:n_gpu]
            self.host[h] = rows[n_gpu:]

    def _append_ring(self, las: np.ndarray, rows: Optional[np.ndarray], free_host: np.ndarray) -> None:
        """Placement "ring" (an alternative reading of who places new KV, section 2;
        section 3: entries of the current round stay on the GPU): in list order,
        each entry takes the next slot of the step's victim order (free ascending,
        then cold, then the ring from the oldest bucket to the newest, never the
        current bucket) and joins the current bucket, the round the last step
        used; an entry that held that slot moves to the lowest free host slot
        (its rows with it). Entries placed later in the same call cannot take
        earlier ones' slots (the current bucket is never a victim). Once no
        victim is left, entries take the lowest free host slots. Taking the next
        victim one entry at a time is taking the first q of the order at once,
        q = min(n, victims available); every eviction comes before every
        host-placed entry, so evicted entries take the lowest free host slots
        in victim order and the host-placed entries the next ones."""
        n = las.size
        cand = np.concatenate([np.flatnonzero(b) for b in self._victim_order()])
        q = min(n, cand.size)
        V = cand[:q]
        owners = self.gown[V].astype(np.int64)
        ev = owners != -1
        n_ev = int(ev.sum())
        h_ev = free_host[:n_ev]
        h_new = free_host[n_ev:n_ev + (n - q)]
        # the data first: the evicted rows to the host, the appended rows in
        if self.full_data:
            self.host[h_ev] = self.gpu[V[ev]]
            self.gpu[V] = rows[:q]
            self.host[h_new] = rows[q:]
        # then the mapping table and owners
        self.map[owners[ev]] = HOST_BIT | h_ev.astype(np.uint32)
        self.hown[h_ev] = owners[ev]
        self.map[las[:q]] = V.astype(np.uint32)
        self.gown[V] = las[:q]
        self.map[las[q:]] = HOST_BIT | h_new.astype(np.uint32)
        self.hown[h_new] = las[q:]
        # the taken slots join the current bucket
        self.free[V] = False
        self.cold[V] = False
        self.ring[:, V] = False
        self.ring[self.cur, V] = True

    # ------------------------------------------------------------------
    def release(self, las: np.ndarray) -> None:
        """Give back the slots of finished entries (section 1: in a shared pool the
        space one request frees serves the others; section 2: placement is the
        library's).

        Reading: every released address must be appended and listed once; it
        becomes absent (it may be appended again); its GPU slot leaves whatever
        bucket holds it and becomes free, or its host slot becomes free. Nothing
        else changes (the ring, ``cur``, ``flag`` and the statistics stay).
        """
        las = np.asarray(las, dtype=np.int64).reshape(-1)
        if las.size == 0:
            return
        if las.min() < 0 or las.max() >= self.N:
            raise OracleError("ERANGE", "address out of range")
        if np.unique(las).size != las.size:
            raise OracleError("EDUP", "address repeated in one release")
        loc = self.map[las]
        if (loc == ABSENT).any():
            raise OracleError("ERANGE", "address not appended")
        on_gpu = (loc & HOST_BIT) == 0
        s = loc[on_gpu].astype(np.int64)
        self.cold[s] = False
        self.ring[:, s] = False
        self.free[s] = True
        self.gown[s] = -1
        h = (loc[~on_gpu] & ~HOST_BIT).astype(np.int64)
        self.hown[h] = -1
        self.map[las] = ABSENT

    # ------------------------------------------------------------------
    def step(self, sel: np.ndarray) -> StepStats:
        """One scheduling round of this group over its selection sets."""
        sel = np.asarray(sel, dtype=np.int64)
        flat = sel.reshape(-1)
        t = self.flag + 1

        # S1 validate: -1 padding, else an appended address in [0, N)
        valid = flat != -1
        v = flat[valid]
        if v.size and (v.min() < 0 or v.max() >= self.N):
            raise OracleError("ERANGE", "selected address out of range")
        if v.size and (self.map[v] == ABSENT).any():
            raise OracleError("ERANGE", "selected address never appended")

        # S2 de-duplicate once for the whole group (section 2)
        U = self._dedup(v)
        invalid = int(flat.size - v.size)

        # S3 lookup through the mapping table (section 2)
        loc = self.map[U]
        on_host = (loc & HOST_BIT) != 0
        hit_slots = loc[~on_host].astype(np.int64)
        miss_la = U[on_host]
        miss_h = (loc[on_host] & ~HOST_BIT).astype(np.int64)

        # S4 capacity: the current bucket is never evicted, so every unique entry
        # needs its own GPU slot (reading: an error that changes nothing)
        if U.size > self.P:
            raise OracleError("ECAPACITY", "more unique entries than GPU slots")

        # S5 the ring index moves on; slots still labelled with the reused
        # bucket become cold, a relabelling only (section 3)
        self.cur = (self.cur + 1) % self.B
        self.cold |= self.ring[self.cur]
        self.ring[self.cur] = False

        # S6 hit marking: a hit slot leaves its bucket and joins the current one
        # (hit slots are distinct, so the order of these updates is immaterial)
        self.cold[hit_slots] = False
        self.ring[:, hit_slots] = False
        self.ring[self.cur, hit_slots] = True

        # S7 victims: ascending slot order inside each bucket, buckets in the
        # order of _victim_order (section 3)
        candidates = np.concatenate([np.flatnonzero(b) for b in self._victim_order()])
        m = miss_la.size
        victims = candidates[:m]
        assert victims.size == m   # guaranteed by S4: |free|+|cold|+|other rings| >= P - |hits| >= m

        # S8 rows before the table (section 3): the missed rows come from the host,
        # the victims' rows go to the host slot the miss vacated. Pairs are
        # disjoint (distinct victims, distinct host slots), so the moves commute.
        owners = self.gown[victims].astype(np.int64)
        evict = owners != -1
        if self.full_data:
            tmp = self.gpu[victims].copy()
            self.gpu[victims] = self.host[miss_h]
            self.host[miss_h[evict]] = tmp[evict]

        # S9 then update the mapping table and owners (section 3)
        self.map[miss_la] = victims.astype(np.uint32)
        self.gown[victims] = miss_la
        self.map[owners[evict]] = HOST_BIT | miss_h[evict].astype(np.uint32)
        self.hown[miss_h[evict]] = owners[evict]
        self.hown[miss_h[~evict]] = -1
        # the loaded slots join the current bucket
        self.free[victims] = False
        self.cold[victims] = False
        self.ring[:, victims] = False
        self.ring[self.cur, victims] = True

        # S10 signal completion
        self.flag = t
        n_free = int((~evict).sum())
        self.last = StepStats(unique=int(U.size), hits=int(hit_slots.size), misses=int(m),
                              evictions=int(m - n_free), from_free=n_free, invalid=invalid)
        self.last_lists = (U, hit_slots, miss_la, miss_h, victims)
        return self.last

    # ------------------------------------------------------------------
    def _dedup(self, v: np.ndarray) -> np.ndarray:
        """S2: the distinct valid addresses of a step in first-occurrence order
        over (set, index), row-major (the reading of "once for such a group")."""
        _, first = np.unique(v, return_index=True)
        return v[np.sort(first)]

    def _victim_order(self) -> list:
        """S7: the buckets victims come from, in order: free, then cold, then the
        ring from the oldest bucket (cur+1) to the newest (cur-1); the current
        bucket never (section 3)."""
        order = [self.free, self.cold]
        order += [self.ring[(self.cur + j) % self.B] for j in range(1, self.B)]
        return order

    # ------------------------------------------------------------------
    def gather(self, sel: np.ndarray, layer: int, step: Optional[int] = None) -> np.ndarray:
        """Rows of one layer for every selected entry, uint8 [n_sets][k][row_bytes].

        Attention reads the selected entries at their (new) GPU locations only
        after the completion signal (section 3). Reading: ``-1`` gives a zero
        row; an entry not GPU-resident, or a gather of a step that has not
        completed, is an error.
        """
        if not self.full_data:
            raise OracleError("EINVAL", "gather needs full-data mode")
        if step is not None and step != self.flag:
            raise OracleError("ENOTRESIDENT", "gather of a step that has not completed")
        if not (0 <= layer < self.layers):
            raise OracleError("EINVAL", "layer out of range")
        sel = np.asarray(sel, dtype=np.int64)
        out = np.zeros(sel.shape + (self.row_bytes,), dtype=np.uint8)
        valid = sel != -1
        la = sel[valid]
        if la.size and (la.min() < 0 or la.max() >= self.N):
            raise OracleError("ERANGE", "gathered address out of range")
        loc = self.map[la]
        if (loc & HOST_BIT).any():    # also catches ABSENT
            raise OracleError("ENOTRESIDENT", "gathered entry is not on the GPU")
        out[valid] = self.gpu[loc.astype(np.int64), layer]
        return out

    # ------------------------------------------------------------------
    def bitsets(self) -> np.ndarray:
        """uint32 [B+2][ceil(P/32)]: free, cold, ring[0], ..., ring[B-1]."""
        return np.stack([pack_bits(self.free), pack_bits(self.cold)]
                        + [pack_bits(self.ring[b]) for b in range(self.B)])

    def export_state(self) -> dict:
        return dict(map=self.map.copy(), gown=self.gown.copy(), hown=self.hown.copy(),
                    bitsets=self.bitsets(), cur=int(self.cur), flag=int(self.flag),
                    stats=self.last.as_tuple())

    def read_row(self, la: int) -> np.ndarray:
        """The stored rows [layers][row_bytes] of one entry, wherever it lives."""
        loc = self.map[la]
        if loc == ABSENT:
            raise OracleError("ERANGE", "never appended")
        if loc & HOST_BIT:
            return self.host[int(loc & ~HOST_BIT)].copy()
        return self.gpu[int(loc)].copy()
