"""Seeded decode traces: initial load order, per-step appends and selections.

The pages describe sparse attention that picks a small top-k subset of past
positions at every decoding step, with heavy overlap between consecutive steps
(UlaCache summary, intro and section 2). The generator below draws such sets:

* step 1: every set draws ``k`` distinct positions by the new-pick rule;
* step t > 1: a set keeps ``floor(overlap * k)`` entries of its previous set,
  chosen uniformly without replacement, and draws the rest by the new-pick
  rule; duplicates are redrawn; every set is stored in ascending order;
* new-pick rule: with probability ``p_recent`` a position uniform in
  ``[L - window, L)``, otherwise uniform in ``[0, L)``, where ``L`` is the
  request's length after the step's appends (appends come before the step's
  selection, so a freshly appended position can be selected at once);
* speculative verify (3 sets per request): set 0 follows the rule above from
  the previous base set; each draft set keeps ``floor(draft_keep * k)``
  entries of the base set and draws the rest by the new-pick rule. Sets are
  stored request-major, ``[r * 3 + d]``.

Logical addresses are ``base_r + position`` with
``base_r = sum_{r' < r} (L_r' + steps * appends)``, so every position a trace
will ever append has its address reserved up front.

Initial residency: the GPU pool starts full. It receives each request's most
recent ``floor(P / R)`` positions (the first ``P mod R`` requests get one
more), appended oldest first in (age descending, request ascending) order so
that slot 0 holds the oldest. The rest of the history is appended afterwards
in (request ascending, position ascending) order and lands in the host pool.
"""

from __future__ import annotations

from typing import Iterator, Optional

import numpy as np

from .configs import Workload, _frac_count


class Trace:
    def __init__(self, wl: Workload, steps: Optional[int] = None):
        self.wl = wl
        self.steps = wl.steps if steps is None else int(steps)
        self.L = wl.lengths()                                   # int64 [R]
        span = self.L + self.steps * wl.appends
        self.base = np.concatenate([[0], np.cumsum(span)[:-1]]).astype(np.int64)
        self.N = int(span.sum())
        self.P = wl.gpu_slots()
        self.H = self.N - self.P
        self.n_sets = wl.n_sets()
        self.k = wl.k
        if self.N >= 2 ** 31:
            raise ValueError("logical capacity must stay below 2^31")
        if int(self.L.min()) < wl.k:
            raise ValueError("every context must hold at least k positions")

    # ---- loads and appends --------------------------------------------
    def initial_load_order(self) -> np.ndarray:
        """All initial-history logical addresses in append order (int32)."""
        R, P, L, base = self.wl.requests, self.P, self.L, self.base
        per = np.full(R, P // R, dtype=np.int64)
        per[: P % R] += 1
        per = np.minimum(per, L)
        # resident part: age a = L_r - 1 - position, order (age desc, request asc)
        amax = int(per.max()) if R else 0
        ages = np.arange(amax - 1, -1, -1, dtype=np.int64)           # descending
        req = np.arange(R, dtype=np.int64)
        A, Rr = np.meshgrid(ages, req, indexing="ij")                 # [amax][R]
        keep = A < per[Rr]
        resident = (base[Rr] + L[Rr] - 1 - A)[keep]
        # host part: request asc, position asc, positions [0, L_r - per_r)
        host = np.concatenate([base[r] + np.arange(L[r] - per[r], dtype=np.int64) for r in range(R)])
        return np.concatenate([resident, host]).astype(np.int32)

    def appends(self, t: int) -> np.ndarray:
        """Logical addresses appended before step t (1-based), request asc."""
        a = self.wl.appends
        out = []
        for r in range(self.wl.requests):
            p0 = int(self.L[r]) + a * (t - 1)
            out.append(self.base[r] + np.arange(p0, p0 + a, dtype=np.int64))
        return np.concatenate(out).astype(np.int32)

    # ---- selections ------------------------------------------------------
    def _new_picks(self, rng, n: int, length: int, exclude: np.ndarray) -> np.ndarray:
        wl = self.wl
        out = np.empty(0, dtype=np.int64)
        lo_recent = max(length - wl.window, 0)
        while out.size < n:
            m = n - out.size
            m2 = m + m // 4 + 8
            recent = rng.random(m2) < wl.p_recent
            lo = np.where(recent, lo_recent, 0)
            cand = rng.integers(lo, length)
            cand = cand[~np.isin(cand, exclude)]
            cand = cand[~np.isin(cand, out)]
            _, first = np.unique(cand, return_index=True)
            cand = cand[np.sort(first)]
            out = np.concatenate([out, cand[:m]])
        return out

    def selections(self, g: int) -> Iterator[np.ndarray]:
        """Yield int32 [n_sets][k] selected logical addresses for t = 1..steps."""
        wl, k = self.wl, self.k
        rng = np.random.default_rng([wl.seed, 1 + g])
        nkeep = _frac_count(wl.overlap, k)
        dkeep = _frac_count(wl.draft_keep, k)
        S = wl.sets_per_request
        prev = [None] * wl.requests
        for t in range(1, self.steps + 1):
            sel = np.empty((self.n_sets, k), dtype=np.int32)
            for r in range(wl.requests):
                length = int(self.L[r]) + wl.appends * t
                if prev[r] is None:
                    cur = self._new_picks(rng, k, length, np.empty(0, dtype=np.int64))
                else:
                    keep = rng.choice(prev[r], size=nkeep, replace=False)
                    cur = np.concatenate([keep, self._new_picks(rng, k - nkeep, length, keep)])
                cur.sort()
                prev[r] = cur
                sel[r * S] = (cur + self.base[r]).astype(np.int32)
                for d in range(1, S):
                    keep = rng.choice(cur, size=dkeep, replace=False)
                    dset = np.concatenate([keep, self._new_picks(rng, k - dkeep, length, keep)])
                    dset.sort()
                    sel[r * S + d] = (dset + self.base[r]).astype(np.int32)
            yield sel

    def all_selections(self, g: int) -> np.ndarray:
        """int32 [steps][n_sets][k]."""
        return np.stack(list(self.selections(g)))
