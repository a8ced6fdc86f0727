"""Invariants of the oracle state after every step of random tiny traces.

I1 an entry is on the GPU or on the host, never both (UlaCache summary, section 2);
I2 free, cold and ring buckets partition the GPU slots (section 3);
I3 after a step the current bucket is exactly the step's unique entries;
I4 no victim comes from the current bucket (section 3);
I5 eviction starts only once the GPU pool is full; I6 conservation of counts;
I7 every stored row equals its closed form; I8 gathered rows equal their closed
form or zeros for padding; I9 the completion counter equals the step number.
"""

import numpy as np
import pytest

from oracle.invariants import check_state, check_step
from oracle.pblru import PBLRUGroup
from synth import Trace, rows_for

from tracegen import padded_selections, tiny_workload


@pytest.mark.parametrize("seed", range(30))
def test_invariants_random(seed):
    wl = tiny_workload(seed)
    tr = Trace(wl)
    g = PBLRUGroup(tr.N, tr.P, tr.H, wl.ring, wl.layers, wl.row_bytes, full_data=True)
    load = tr.initial_load_order()
    g.append(load, rows_for(wl.seed, 0, load, wl.layers, wl.row_bytes))
    check_state(g.export_state(), tr.P, tr.H)
    for t, sel in enumerate(padded_selections(tr, 0, seed), 1):
        app = tr.appends(t)
        g.append(app, rows_for(wl.seed, 0, app, wl.layers, wl.row_bytes))
        prev = g.export_state()
        g.step(sel)
        st = g.export_state()
        U, hit_slots, _, _, victims = g.last_lists
        check_step(prev, st, tr.P, tr.H, U=U, victims=victims, hit_slots=hit_slots)
        assert st["flag"] == t                                   # I9
        # I7: every appended entry holds its own rows wherever it lives
        appended = np.flatnonzero(g.map != 0xFFFFFFFF)
        want = rows_for(wl.seed, 0, appended, wl.layers, wl.row_bytes)
        got = np.stack([g.read_row(int(la)) for la in appended])
        assert (got == want).all()
        # I8: gathered rows
        for layer in range(wl.layers):
            out = g.gather(sel, layer, step=t)
            valid = sel != -1
            assert (out[~valid] == 0).all()
            ref = rows_for(wl.seed, 0, sel[valid], wl.layers, wl.row_bytes)[:, layer]
            assert (out[valid] == ref).all()


@pytest.mark.parametrize("seed", range(16))
def test_invariants_ring_placement(seed):
    """I1-I9 with appends placed in the current bucket: after every append (I1, I2:
    the evicted entries moved to the host, nothing held twice) and every step,
    stored and gathered rows against their closed form."""
    wl = tiny_workload(seed, steps=10)
    tr = Trace(wl)
    g = PBLRUGroup(tr.N, tr.P, tr.H, wl.ring, wl.layers, wl.row_bytes, full_data=True, placement="ring")
    load = tr.initial_load_order()
    g.append(load, rows_for(wl.seed, 0, load, wl.layers, wl.row_bytes))
    check_state(g.export_state(), tr.P, tr.H)
    for t, sel in enumerate(padded_selections(tr, 0, seed), 1):
        app = tr.appends(t)
        g.append(app, rows_for(wl.seed, 0, app, wl.layers, wl.row_bytes))
        check_state(g.export_state(), tr.P, tr.H)
        prev = g.export_state()
        g.step(sel)
        st = g.export_state()
        U, hit_slots, _, _, victims = g.last_lists
        check_step(prev, st, tr.P, tr.H, U=U, victims=victims, hit_slots=hit_slots)
        appended = np.flatnonzero(g.map != 0xFFFFFFFF)
        want = rows_for(wl.seed, 0, appended, wl.layers, wl.row_bytes)
        assert (np.stack([g.read_row(int(la)) for la in appended]) == want).all()
        for layer in range(wl.layers):
            out = g.gather(sel, layer, step=t)
            valid = sel != -1
            assert (out[valid] == rows_for(wl.seed, 0, sel[valid], wl.layers, wl.row_bytes)[:, layer]).all()


@pytest.mark.parametrize("seed", range(12))
def test_invariants_hold_with_releases(seed):
    """I1-I9 after every step of traces whose finished entries are released between
    steps (released addresses are absent; their slots are free, so later misses take
    free GPU slots first and free host slots are reused by appends)."""
    from tracegen import release_plan
    wl = tiny_workload(seed, steps=10)
    tr = Trace(wl)
    sels = padded_selections(tr, 0, seed)
    plan = release_plan(tr, sels, seed, frac=0.4)
    g = PBLRUGroup(tr.N, tr.P, tr.H, wl.ring, wl.layers, wl.row_bytes, full_data=True)
    load = tr.initial_load_order()
    g.append(load, rows_for(wl.seed, 0, load, wl.layers, wl.row_bytes))
    for t, sel in enumerate(sels, 1):
        app = tr.appends(t)
        g.append(app, rows_for(wl.seed, 0, app, wl.layers, wl.row_bytes))
        prev = g.export_state()
        g.step(sel)
        st = g.export_state()
        U, hit_slots, _, _, victims = g.last_lists
        check_step(prev, st, tr.P, tr.H, U=U, victims=victims, hit_slots=hit_slots)
        appended = np.flatnonzero(g.map != 0xFFFFFFFF)
        want = rows_for(wl.seed, 0, appended, wl.layers, wl.row_bytes)
        assert (np.stack([g.read_row(int(la)) for la in appended]) == want).all()
        for layer in range(wl.layers):
            out = g.gather(sel, layer, step=t)
            valid = sel != -1
            assert (out[valid] == rows_for(wl.seed, 0, sel[valid], wl.layers, wl.row_bytes)[:, layer]).all()
        rel = plan.get(t, np.zeros(0, np.int32))
        g.release(rel)
        assert (g.map[rel] == 0xFFFFFFFF).all()
        check_state(g.export_state(), tr.P, tr.H)


def test_release_errors_change_nothing():
    from oracle.pblru import OracleError
    wl = tiny_workload(1)
    tr = Trace(wl)
    g = PBLRUGroup(tr.N, tr.P, tr.H, wl.ring, wl.layers, wl.row_bytes, full_data=False)
    g.append(tr.initial_load_order(), None)
    st = g.export_state()
    first = int(tr.initial_load_order()[0])
    never = int(tr.appends(1)[0]) if tr.appends(1).size else tr.N
    for bad, name in [([tr.N], "ERANGE"), ([-1], "ERANGE"), ([never], "ERANGE"), ([first, first], "EDUP")]:
        with pytest.raises(OracleError) as e:
            g.release(np.array(bad, dtype=np.int64))
        assert e.value.name == name
        after = g.export_state()
        for k in ("map", "gown", "hown", "bitsets"):
            assert np.array_equal(after[k], st[k])
