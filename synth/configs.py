"""Workload presets: sizes of the synthetic decode traces.

Each preset fixes the request count and context lengths, the number of layer
groups and layers per group, the per-step top-k, the GPU pool size, the ring
length, the step count and the selection statistics. Readings that the pages
leave open are fixed here and stated next to the field that carries them:

* the GPU pool of a group holds ``floor(pool_frac * total history)`` slots and
  the host pool holds every other logical entry the trace will ever append,
  so ``host_slots = logical_capacity - gpu_slots``;
* workloads that do not say how many layers share a selection use one layer
  per group; those that do not say how many positions a step appends use one
  per request (one token per decode step);
* the speculative-verify workload appends three positions per request every
  step (every step is treated as accepted).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    requests: int
    ctx_fixed: Optional[int]            # every request has this many history positions
    ctx_range: Optional[Tuple[int, int]]  # else uniform integer in [lo, hi] inclusive
    sets_per_request: int               # 1, or 3 for base + 2 draft tokens
    draft_keep: float                   # share of the base set each draft set keeps
    groups: int
    layers: int                         # layers per group sharing one selection
    k: int                              # positions selected per set
    pool_frac: float                    # GPU pool = floor(pool_frac * total history)
    pool_slots: Optional[int]           # explicit GPU pool size (overrides pool_frac)
    ring: int                           # ring buckets per group
    steps: int
    appends: int                        # positions appended per request per step
    overlap: float                      # share of the previous set kept each step
    p_recent: float                     # probability that a new pick is from the recent window
    window: int                         # recent window length
    row_bytes: int = 656                # 512 FP8 latent + 64 bf16 rope + 16 B scales
    seed: int = 0

    # ---- derived sizes -------------------------------------------------
    def lengths(self) -> np.ndarray:
        """Initial history length of every request (int64)."""
        if self.ctx_fixed is not None:
            return np.full(self.requests, self.ctx_fixed, dtype=np.int64)
        lo, hi = self.ctx_range
        rng = np.random.default_rng([self.seed, 0xC0])
        return rng.integers(lo, hi, endpoint=True, size=self.requests).astype(np.int64)

    def history(self) -> int:
        return int(self.lengths().sum())

    def logical_capacity(self, steps: Optional[int] = None) -> int:
        s = self.steps if steps is None else steps
        return int((self.lengths() + s * self.appends).sum())

    def gpu_slots(self) -> int:
        if self.pool_slots is not None:
            return int(self.pool_slots)
        return int(np.floor(self.pool_frac * self.history()))

    def host_slots(self, steps: Optional[int] = None) -> int:
        return self.logical_capacity(steps) - self.gpu_slots()

    def n_sets(self) -> int:
        return self.requests * self.sets_per_request


def _frac_count(frac: float, k: int) -> int:
    """floor(frac * k) without binary-float surprises (frac has <= 4 decimals)."""
    return (int(round(frac * 10000)) * k) // 10000


PRESETS = {
    # 4 requests x 4096 positions, one group of one layer, seed 0.
    "tiny_4x4k": Workload(
        name="tiny_4x4k", requests=4, ctx_fixed=4096, ctx_range=None, sets_per_request=1,
        draft_keep=0.0, groups=1, layers=1, k=256, pool_frac=0.5, pool_slots=8192, ring=4,
        steps=8, appends=1, overlap=0.8, p_recent=0.5, window=1024),
    # 16 requests x 64K, one group of 3 layers sharing one selection.
    "r16_64k_g1x3": Workload(
        name="r16_64k_g1x3", requests=16, ctx_fixed=65536, ctx_range=None, sets_per_request=1,
        draft_keep=0.0, groups=1, layers=3, k=2048, pool_frac=0.5, pool_slots=None, ring=8,
        steps=64, appends=1, overlap=0.85, p_recent=0.7, window=4096),
    # 64 requests, contexts U[64K,128K], 24 groups x 3 layers with independent selections.
    "r64_64k128k_g24x3": Workload(
        name="r64_64k128k_g24x3", requests=64, ctx_fixed=None, ctx_range=(65536, 131072),
        sets_per_request=1, draft_keep=0.0, groups=24, layers=3, k=2048, pool_frac=0.25,
        pool_slots=None, ring=8, steps=32, appends=1, overlap=0.85, p_recent=0.7, window=4096),
    # Speculative verify: 128 requests x 3 sets (base + 2 drafts), 4 groups.
    "spec3_r128_64k128k_g4": Workload(
        name="spec3_r128_64k128k_g4", requests=128, ctx_fixed=None, ctx_range=(65536, 131072),
        sets_per_request=3, draft_keep=0.9, groups=4, layers=1, k=2048, pool_frac=0.25,
        pool_slots=None, ring=8, steps=32, appends=3, overlap=0.85, p_recent=0.7, window=4096),
    # Eviction stress: 256 x 128K, pool 10%, 16-bucket ring, 50% overlap, uniform picks.
    "evict_r256_128k_g2": Workload(
        name="evict_r256_128k_g2", requests=256, ctx_fixed=131072, ctx_range=None,
        sets_per_request=1, draft_keep=0.0, groups=2, layers=1, k=2048, pool_frac=0.1,
        pool_slots=None, ring=16, steps=16, appends=1, overlap=0.5, p_recent=0.0, window=4096),
    # Its control: 98% overlap, almost no eviction.
    "evict_r256_128k_g2_ctl98": Workload(
        name="evict_r256_128k_g2_ctl98", requests=256, ctx_fixed=131072, ctx_range=None,
        sets_per_request=1, draft_keep=0.0, groups=2, layers=1, k=2048, pool_frac=0.1,
        pool_slots=None, ring=16, steps=16, appends=1, overlap=0.98, p_recent=0.0, window=4096),
}


def preset(name: str) -> Workload:
    return PRESETS[name]


def scaled(wl: Workload, factor: int, **overrides) -> Workload:
    """The same structure at 1/factor of the context, top-k and window sizes.

    Request counts, groups, layers, ring length, steps and selection
    statistics are kept; the GPU pool keeps its share of the history.
    """
    def div(x):
        return max(1, x // factor)

    kw = dict(
        name=f"{wl.name}_div{factor}",
        ctx_fixed=None if wl.ctx_fixed is None else div(wl.ctx_fixed),
        ctx_range=None if wl.ctx_range is None else (div(wl.ctx_range[0]), div(wl.ctx_range[1])),
        k=div(wl.k),
        window=div(wl.window),
        pool_slots=None if wl.pool_slots is None else div(wl.pool_slots),
    )
    kw.update(overrides)
    return dataclasses.replace(wl, **kw)
