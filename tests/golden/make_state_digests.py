"""Write tests/golden/digests_<workload>.json from the CPU oracle only.

For every workload preset, every layer group and every step, the oracle (in
metadata mode: mapping table, owners, buckets, no row bytes) replays the seeded
synthetic trace and the digest of its exported state is stored: after the
initial load (step 0) and after each step. The GPU parity tests replay the same
inputs through the engine and compare digests. With --lru the exact-LRU oracle
(array form) replays the same traces into digests_lru_<workload>.json, with the
timestamps in the digest. With --ring the PB-LRU oracle places appended
entries in the current bucket (placement "ring") and writes
digests_ring_<workload>.json. Usage:

    python tests/golden/make_state_digests.py [--lru | --ring] [workload ...]
"""

import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

from digests import digest  # noqa: E402
from oracle.replay import initial_load, new_group  # noqa: E402
from synth import PRESETS, Trace, preset  # noqa: E402


def lru_group_digests(name: str, g: int) -> list:
    from oracle.exact_lru_np import ExactLRUArrays
    tr = Trace(preset(name))
    grp = ExactLRUArrays(tr.N, tr.P, tr.H, tr.wl.ring)
    grp.append(tr.initial_load_order())
    out = [digest(grp.export_state())]
    sels = tr.selections(g)
    for t in range(1, tr.steps + 1):
        grp.append(tr.appends(t))
        grp.step(next(sels))
        out.append(digest(grp.export_state()))
    return out


def group_digests(name: str, g: int, placement: str = "lowest") -> list:
    tr = Trace(preset(name))
    grp = new_group(tr, full_data=False, placement=placement)
    initial_load(grp, tr, g)
    out = [digest(grp.export_state())]
    sels = tr.selections(g)
    for t in range(1, tr.steps + 1):
        grp.append(tr.appends(t), None)
        grp.step(next(sels))
        out.append(digest(grp.export_state()))
    return out


def ring_group_digests(name: str, g: int) -> list:
    return group_digests(name, g, placement="ring")


def main(names, lru=False, ring=False):
    jobs = [(n, g) for n in names for g in range(preset(n).groups)]
    fn = lru_group_digests if lru else (ring_group_digests if ring else group_digests)
    with ProcessPoolExecutor(max_workers=min(6, len(jobs))) as ex:
        res = list(ex.map(fn, [j[0] for j in jobs], [j[1] for j in jobs]))
    by = {}
    for (n, g), d in zip(jobs, res):
        by.setdefault(n, {})[g] = d
    for n in names:
        wl = preset(n)
        doc = {"workload": n, "policy": "exact LRU" if lru else "PB-LRU",
               "placement": "ring" if ring else "lowest",
               "source": ("oracle/exact_lru_np.py" if lru else "oracle/ (metadata mode)")
               + " via tests/golden/make_state_digests.py",
               "digest": "xxh3_64 of the little-endian bytes of map, gown, hown, bitsets"
               + (", stamps" if lru else ""),
               "steps": wl.steps, "groups": [by[n][g] for g in range(wl.groups)]}
        fname = f"digests_lru_{n}.json" if lru else (f"digests_ring_{n}.json" if ring else f"digests_{n}.json")
        with open(os.path.join(HERE, fname), "w") as f:
            json.dump(doc, f, separators=(",", ":"))
        print("wrote", n, flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    lru = "--lru" in args
    ring = "--ring" in args
    names = [a for a in args if a not in ("--lru", "--ring")]
    main(names or list(PRESETS), lru=lru, ring=ring)
