"""Planted mistakes in the PB-LRU oracle (test infrastructure only).

Each class is the oracle with one plausible implementation error, so the tests
can show that the pins and checkers which are supposed to catch that error do
catch it. None of them is used outside the tests that expect them to fail.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from oracle.pblru import PBLRUGroup


class AddressOrderDedup(PBLRUGroup):
    """De-duplication in ascending address order instead of first occurrence
    (UlaCache summary, section 2: the order then depends on address values,
    which the policy must never look at)."""

    def _dedup(self, v):
        return np.unique(v)


class RepeatsCountedAsAccesses(PBLRUGroup):
    """Hits and misses counted per selection entry instead of per distinct
    entry, so a repeated read inside one step counts twice."""

    def step(self, sel):
        st = super().step(sel)
        flat = np.asarray(sel, dtype=np.int64).reshape(-1)
        v = flat[flat != -1]
        U, _, miss_la, _, _ = self.last_lists
        missed = np.isin(v, miss_la)
        self.last = dataclasses.replace(st, unique=int(v.size), hits=int((~missed).sum()),
                                        misses=int(missed.sum()))
        return self.last


class PaddingMovesRing(PBLRUGroup):
    """A step whose selection contains padding advances the ring one extra
    position (padding treated as a round of its own)."""

    def step(self, sel):
        if (np.asarray(sel) == -1).any():
            self.cur = (self.cur + 1) % self.B
        return super().step(sel)


class ColdBeforeFree(PBLRUGroup):
    """Victims from the cold bucket before the free slots (section 3 takes the
    free slots first, so eviction begins only once the pool is full)."""

    def _victim_order(self):
        order = super()._victim_order()
        return [order[1], order[0]] + order[2:]


class CurrentBucketEvictable(PBLRUGroup):
    """The current bucket (which holds this step's hits) is a victim source right
    after cold (section 3 never evicts it)."""

    def _victim_order(self):
        order = super()._victim_order()
        return order[:2] + [self.ring[self.cur]] + order[2:]
