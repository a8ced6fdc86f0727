"""Properties of the synthetic traces (inputs shared by the oracle and the engine)."""

import numpy as np
import pytest

from synth import PRESETS, Trace, preset, scaled
from synth.configs import _frac_count


def test_preset_sizes():
    tr = Trace(preset("tiny_4x4k"))
    assert (tr.N, tr.P, tr.H) == (16416, 8192, 8224)
    tr = Trace(preset("r16_64k_g1x3"))
    assert (tr.N, tr.P) == (1049600, 524288)
    assert preset("evict_r256_128k_g2").gpu_slots() == 3355443


@pytest.mark.parametrize("name", ["tiny_4x4k", "r16_64k_g1x3", "spec3_r128_64k128k_g4"])
def test_selection_properties(name):
    wl = scaled(preset(name), 16) if name != "tiny_4x4k" else preset(name)
    tr = Trace(wl, steps=min(wl.steps, 5))
    S = wl.sets_per_request
    prev = None
    for t, sel in enumerate(tr.selections(0), 1):
        assert sel.shape == (tr.n_sets, wl.k) and sel.dtype == np.int32
        for j in range(tr.n_sets):
            r = j // S
            pos = sel[j].astype(np.int64) - tr.base[r]
            assert (np.diff(pos) > 0).all()                       # sorted, distinct
            assert pos.min() >= 0 and pos.max() < tr.L[r] + wl.appends * t
            if S == 3 and j % S:
                base = sel[r * S]
                assert np.intersect1d(base, sel[j]).size >= _frac_count(wl.draft_keep, wl.k)
        if prev is not None:
            for r in range(wl.requests):
                kept = np.intersect1d(prev[r * S], sel[r * S]).size
                assert kept >= _frac_count(wl.overlap, wl.k)
        prev = sel


def test_initial_load_is_a_permutation_with_recent_positions_first():
    wl = preset("tiny_4x4k")
    tr = Trace(wl)
    order = tr.initial_load_order().astype(np.int64)
    assert np.array_equal(np.sort(order), np.concatenate(
        [tr.base[r] + np.arange(tr.L[r]) for r in range(wl.requests)]))
    resident = order[: tr.P]
    for r in range(wl.requests):
        pos = resident[(resident >= tr.base[r]) & (resident < tr.base[r] + tr.L[r])] - tr.base[r]
        assert np.array_equal(np.sort(pos), np.arange(tr.L[r] - tr.P // wl.requests, tr.L[r]))
    # oldest first: position L-1-age, ages descending
    assert resident[0] == tr.base[0] + tr.L[0] - tr.P // wl.requests
    assert resident[tr.P - 1] == tr.base[wl.requests - 1] + tr.L[wl.requests - 1] - 1


def test_appends_cover_the_reserved_range():
    wl = preset("spec3_r128_64k128k_g4")
    tr = Trace(wl, steps=2)
    a1, a2 = tr.appends(1), tr.appends(2)
    assert a1.size == wl.requests * 3
    assert a1[0] == tr.base[0] + tr.L[0] and a2[0] == tr.base[0] + tr.L[0] + 3


def test_seeded_reproducible():
    wl = scaled(preset("r16_64k_g1x3"), 64)
    a = Trace(wl, steps=3).all_selections(0)
    b = Trace(wl, steps=3).all_selections(0)
    c = Trace(wl, steps=3).all_selections(1)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
