"""Small random workloads for the property and parity tests (inputs only)."""

import numpy as np

from synth import Trace, Workload


def tiny_workload(seed: int, ring: int = None, steps: int = None, sets: int = None,
                  layers: int = None, pool: int = None) -> Workload:
    rng = np.random.default_rng([seed, 77])
    R = int(rng.integers(1, 5))
    ctx = int(rng.integers(40, 120))
    k = int(rng.integers(4, ctx // 4))
    steps = int(rng.integers(3, 10)) if steps is None else steps
    appends = int(rng.integers(0, 3))
    S = (1 if rng.random() < 0.6 else 3) if sets is None else sets
    hist = R * ctx
    if pool is None:   # at least one slot per unique entry a step can select
        pool = int(rng.integers(R * S * k, hist + 1))
    return Workload(
        name=f"rand{seed}", requests=R, ctx_fixed=ctx, ctx_range=None, sets_per_request=S,
        draft_keep=0.5, groups=1, layers=int(rng.integers(1, 4)) if layers is None else layers,
        k=k, pool_frac=0.0, pool_slots=pool, ring=int(rng.integers(1, 6)) if ring is None else ring,
        steps=steps, appends=appends, overlap=float(rng.choice([0.0, 0.5, 0.8])),
        p_recent=0.5, window=16, row_bytes=64, seed=seed % 256)


def with_padding(sel: np.ndarray, rng, frac: float = 0.1) -> np.ndarray:
    """Replace a random share of entries by -1 padding."""
    out = sel.copy()
    out[rng.random(out.shape) < frac] = -1
    return out


def padded_selections(trace: Trace, g: int, seed: int, frac: float = 0.1):
    rng = np.random.default_rng([seed, 99])
    return [with_padding(s, rng, frac) for s in trace.selections(g)]


def release_plan(trace: Trace, sels, seed: int, frac: float = 0.3) -> dict:
    """Addresses to release after each step t (before step t+1's appends): a random
    share `frac` of the entries appended so far that no later step selects, so
    that every later selection stays valid. {t: int32 array}."""
    rng = np.random.default_rng([seed, 123])
    sels = [np.asarray(s).reshape(-1) for s in sels]
    later = [set() for _ in range(len(sels) + 1)]
    for t in range(len(sels) - 1, -1, -1):        # later[t]: selected by step t+1 or after
        later[t] = later[t + 1] | set(int(x) for x in sels[t] if x >= 0)
    alive = set(int(x) for x in trace.initial_load_order())
    plan = {}
    for t in range(1, len(sels)):
        alive |= set(int(x) for x in trace.appends(t))
        cand = sorted(alive - later[t])
        k = int(frac * len(cand))
        pick = rng.choice(np.array(cand, dtype=np.int64), size=k, replace=False) if k else np.zeros(0, np.int64)
        rng.shuffle(pick)
        plan[t] = pick.astype(np.int32)
        alive -= set(int(x) for x in pick)
    return plan
