"""Metamorphic pins of the PB-LRU oracle (UlaCache summary, sections 2-3).

The policy looks at addresses only through the mapping table and at a step's
selection only through its distinct valid entries in first-occurrence order, so:

* relabelling every logical address by a permutation (selections, appends,
  releases alike) relabels the mapping table and the owners the same way and
  changes neither the bucket bitsets, the victims, the ring position nor the
  statistics;
* repeating a step's sets (the repeats come after every first occurrence)
  changes nothing at all;
* inserting padding anywhere changes only the padding count.

A policy that ordered anything by address value, counted repeats or padding as
accesses, or let padding move the ring would fail one of these: the planted
mistakes of tests/oracle_mutants.py (address-ordered de-duplication, repeats
counted as accesses, padding that advances the ring) are each run through the
check meant to catch them, which must fail.
"""

import dataclasses

import numpy as np
import pytest

from oracle.pblru import ABSENT, HOST_BIT, PBLRUGroup
from synth import Trace
from oracle_mutants import AddressOrderDedup, PaddingMovesRing, RepeatsCountedAsAccesses
from tracegen import padded_selections, release_plan, tiny_workload


def _run(tr, load, appends, sels, releases, N, cls=PBLRUGroup):
    wl = tr.wl
    g = cls(N, tr.P, tr.H, wl.ring, wl.layers, wl.row_bytes, full_data=False)
    g.append(load, None)
    hist = []
    for t, sel in enumerate(sels, 1):
        g.append(appends[t - 1], None)
        g.step(sel)
        hist.append((g.export_state(), list(g.last_lists[4])))
        rel = releases.get(t)
        if rel is not None and rel.size:
            g.release(rel)
    return hist


def _relabel_map(m, perm):
    """Mapping table under relabelled addresses: entry perm[a] takes a's location."""
    out = np.full_like(m, ABSENT)
    out[perm] = m
    return out


def _relabel_owners(o, perm):
    o = np.asarray(o, dtype=np.int64)
    return np.where(o >= 0, perm[np.maximum(o, 0)], -1)


def check_relabelling(seed, cls=PBLRUGroup):
    wl = tiny_workload(seed, steps=8)
    tr = Trace(wl)
    sels = padded_selections(tr, 0, seed)
    rel = release_plan(tr, sels, seed, frac=0.3)
    load = tr.initial_load_order()
    apps = [tr.appends(t) for t in range(1, tr.steps + 1)]
    base = _run(tr, load, apps, sels, rel, tr.N, cls)
    perm = np.random.default_rng([seed, 31]).permutation(tr.N)
    f = lambda a: np.where(np.asarray(a) >= 0, perm[np.maximum(np.asarray(a), 0)], -1).astype(np.int32)
    other = _run(tr, f(load), [f(a) for a in apps], [f(s) for s in sels],
                 {t: f(r) for t, r in rel.items()}, tr.N, cls)
    for t, ((a, va), (b, vb)) in enumerate(zip(base, other), 1):
        assert va == vb, f"step {t}: victims"
        assert np.array_equal(_relabel_map(a["map"], perm), b["map"]), f"step {t}: map"
        assert np.array_equal(_relabel_owners(a["gown"], perm), b["gown"]), f"step {t}: gown"
        assert np.array_equal(_relabel_owners(a["hown"], perm), b["hown"]), f"step {t}: hown"
        assert np.array_equal(a["bitsets"], b["bitsets"]), f"step {t}: bitsets"
        assert (a["cur"], a["flag"], a["stats"]) == (b["cur"], b["flag"], b["stats"]), f"step {t}"


def check_repeated_sets(seed, cls=PBLRUGroup):
    wl = tiny_workload(seed, steps=8)
    tr = Trace(wl)
    sels = padded_selections(tr, 0, seed)
    rng = np.random.default_rng([seed, 32])
    load = tr.initial_load_order()
    apps = [tr.appends(t) for t in range(1, tr.steps + 1)]
    base = _run(tr, load, apps, sels, {}, tr.N, cls)
    # every step gets extra sets that repeat random earlier sets of the same step
    rep = []
    for s in sels:
        extra = s[rng.integers(0, s.shape[0], size=int(rng.integers(1, 4)))]
        rep.append(np.concatenate([s, extra]))
    other = _run(tr, load, apps, rep, {}, tr.N, cls)
    for t, ((a, va), (b, vb)) in enumerate(zip(base, other), 1):
        assert va == vb, f"step {t}: victims"
        for k in ("map", "gown", "hown", "bitsets"):
            assert np.array_equal(a[k], b[k]), f"step {t}: {k}"
        sa, sb = a["stats"], b["stats"]
        assert sa[:5] == sb[:5], f"step {t}: stats {sa} vs {sb}"   # padding count may grow


def check_padding(seed, cls=PBLRUGroup):
    wl = tiny_workload(seed, steps=8)
    tr = Trace(wl)
    sels = list(tr.selections(0))
    rng = np.random.default_rng([seed, 33])
    load = tr.initial_load_order()
    apps = [tr.appends(t) for t in range(1, tr.steps + 1)]
    base = _run(tr, load, apps, sels, {}, tr.N, cls)
    padded, added = [], []
    for s in sels:
        n_pad = int(rng.integers(1, 9))
        flat = s.reshape(-1)
        pos = np.sort(rng.integers(0, flat.size + 1, size=n_pad))
        new = np.insert(flat, pos, -1)
        width = new.size // s.shape[0] + 1            # keep whole sets: pad the tail too
        new = np.concatenate([new, np.full(s.shape[0] * width - new.size, -1, new.dtype)])
        padded.append(new.reshape(s.shape[0], width).astype(np.int32))
        added.append(int((new == -1).sum()) - int((flat == -1).sum()))
    other = _run(tr, load, apps, padded, {}, tr.N, cls)
    for t, ((a, va), (b, vb)) in enumerate(zip(base, other), 1):
        assert va == vb, f"step {t}: victims"
        for k in ("map", "gown", "hown", "bitsets"):
            assert np.array_equal(a[k], b[k]), f"step {t}: {k}"
        sa, sb = a["stats"], b["stats"]
        assert sa[:5] == sb[:5] and sb[5] == sa[5] + added[t - 1], f"step {t}: stats {sa} vs {sb}"


@pytest.mark.parametrize("seed", range(12))
def test_relabelling_addresses(seed):
    check_relabelling(seed)


@pytest.mark.parametrize("seed", range(12))
def test_repeated_sets_change_nothing(seed):
    check_repeated_sets(seed)


@pytest.mark.parametrize("seed", range(12))
def test_padding_changes_only_the_padding_count(seed):
    check_padding(seed)


def _failing_seeds(check, cls, seeds=range(12)):
    bad = []
    for seed in seeds:
        try:
            check(seed, cls)
        except AssertionError:
            bad.append(seed)
    return bad


@pytest.mark.parametrize("check,mutant", [
    (check_relabelling, AddressOrderDedup),
    (check_repeated_sets, RepeatsCountedAsAccesses),
    (check_padding, PaddingMovesRing),
], ids=["relabel-vs-address-order-dedup", "repeats-vs-repeats-counted", "padding-vs-padding-moves-ring"])
def test_metamorphic_check_catches_planted_mistake(check, mutant):
    """Each metamorphic check fails on the oracle with the mistake it is meant to
    catch (on most seeds: a seed can lack the situation, e.g. a one-bucket ring
    for the ring mutant or a step with a single miss for the order mutant)."""
    bad = _failing_seeds(check, mutant)
    assert len(bad) >= 6, f"{check.__name__} caught {mutant.__name__} only on seeds {bad}"


@pytest.mark.parametrize("seed", range(8))
def test_exact_lru_relabelling_addresses(seed):
    """The same relabelling property for the array form of exact LRU (victims by
    timestamp and slot, never by address), releases included."""
    from oracle.exact_lru_np import ExactLRUArrays
    wl = tiny_workload(seed, steps=10)
    tr = Trace(wl)
    sels = padded_selections(tr, 0, seed)
    rel = release_plan(tr, sels, seed, frac=0.3)
    load = tr.initial_load_order()
    apps = [tr.appends(t) for t in range(1, tr.steps + 1)]
    perm = np.random.default_rng([seed, 34]).permutation(tr.N)
    f = lambda a: np.where(np.asarray(a) >= 0, perm[np.maximum(np.asarray(a), 0)], -1).astype(np.int32)

    def run(fn):
        g = ExactLRUArrays(tr.N, tr.P, tr.H, wl.ring)
        g.append(fn(load))
        out = []
        for t, sel in enumerate(sels, 1):
            g.append(fn(apps[t - 1]))
            g.step(fn(sel))
            out.append((g.export_state(), [int(v) for v in g.last_victims]))
            r = rel.get(t)
            if r is not None and r.size:
                g.release(fn(r))
        return out

    for t, ((a, va), (b, vb)) in enumerate(zip(run(lambda x: np.asarray(x, np.int32)), run(f)), 1):
        assert va == vb, f"step {t}: victims"
        assert np.array_equal(_relabel_map(a["map"], perm), b["map"]), f"step {t}: map"
        assert np.array_equal(_relabel_owners(a["gown"], perm), b["gown"]), f"step {t}: gown"
        assert np.array_equal(_relabel_owners(a["hown"], perm), b["hown"]), f"step {t}: hown"
        assert np.array_equal(a["stamps"], b["stamps"]) and a["stats"] == b["stats"], f"step {t}"
