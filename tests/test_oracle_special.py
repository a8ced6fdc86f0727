"""Special cases that reduce the oracle to something checkable by other means.

* one-bucket ring: every step folds everything into cold, so the victims are
  the lowest free slots and then the lowest occupied slots outside the step's
  hits (UlaCache summary, section 3, with a ring of length one);
* pool holding every entry: no miss ever happens and the gather is a plain
  fancy index of the pool through the mapping table (section 2);
* error paths: a rejected call changes nothing.
"""

import dataclasses

import numpy as np
import pytest

from oracle.pblru import OracleError, PBLRUGroup
from oracle.replay import replay
from synth import Trace, rows_for

from tracegen import padded_selections, tiny_workload


@pytest.mark.parametrize("seed", range(10))
def test_one_bucket_ring_victims_are_lowest_slots_outside_hits(seed):
    wl = dataclasses.replace(tiny_workload(seed), ring=1)
    tr = Trace(wl)
    g = PBLRUGroup(tr.N, tr.P, tr.H, 1, wl.layers, wl.row_bytes, full_data=False)
    g.append(tr.initial_load_order(), None)
    for t, sel in enumerate(padded_selections(tr, 0, seed), 1):
        g.append(tr.appends(t), None)
        free_before = set(np.flatnonzero(g.gown == -1).tolist())
        g.step(sel)
        U, hit_slots, miss_la, _, victims = g.last_lists
        hits = set(hit_slots.tolist())
        others = [s for s in range(tr.P) if s not in hits and s not in free_before]
        want = (sorted(free_before) + others)[: miss_la.size]
        assert victims.tolist() == want


@pytest.mark.parametrize("seed", range(6))
def test_pool_holds_everything_gather_is_fancy_index(seed):
    wl = tiny_workload(seed)
    tr0 = Trace(wl)
    wl = dataclasses.replace(wl, pool_slots=tr0.N)
    tr = Trace(wl)
    for t, sel, g, outs in replay(tr, 0, selections=padded_selections(tr, 0, seed)):
        assert g.last.misses == 0 and g.last.hits == g.last.unique
        valid = sel != -1
        for layer, out in enumerate(outs):
            ref = np.zeros_like(out)
            ref[valid] = g.gpu[g.map[sel[valid]].astype(np.int64), layer]
            assert (out == ref).all()


def _small():
    wl = tiny_workload(3, ring=3)
    tr = Trace(wl)
    g = PBLRUGroup(tr.N, tr.P, tr.H, wl.ring, wl.layers, wl.row_bytes, full_data=True)
    load = tr.initial_load_order()
    g.append(load, rows_for(wl.seed, 0, load, wl.layers, wl.row_bytes))
    return wl, tr, g


def _same(a, b):
    return all(np.array_equal(np.asarray(a[k]), np.asarray(b[k])) for k in a)


def test_errors_leave_state_unchanged():
    wl, tr, g = _small()
    before = g.export_state()
    cases = [
        ("ERANGE", lambda: g.step(np.array([[0, tr.N]]))),
        ("ERANGE", lambda: g.step(np.array([[-2]]))),
        ("ERANGE", lambda: g.step(np.array([[tr.appends(1)[0]]]))),     # never appended
        ("ECAPACITY", lambda: g.step(np.arange(tr.P + 1)[None, :])),
        ("EDUP", lambda: g.append(np.array([0]), np.zeros((1, wl.layers, wl.row_bytes)))),
        ("EDUP", lambda: g.append(np.array([tr.appends(1)[0]] * 2), np.zeros((2, wl.layers, wl.row_bytes)))),
        ("ERANGE", lambda: g.append(np.array([tr.N]), np.zeros((1, wl.layers, wl.row_bytes)))),
        ("ENOTRESIDENT", lambda: g.gather(np.array([[int(np.flatnonzero(g.map & 0x80000000 != 0)[0])]]), 0)),
        ("ENOTRESIDENT", lambda: g.gather(np.array([[0]]), 0, step=5)),
    ]
    for name, fn in cases:
        with pytest.raises(OracleError) as e:
            fn()
        assert e.value.name == name
        assert _same(before, g.export_state())


def test_host_full_append_rejected():
    g = PBLRUGroup(N=10, P=2, H=2, B=2, layers=1, row_bytes=16, full_data=False)
    g.append(np.arange(4), None)
    before = g.export_state()
    with pytest.raises(OracleError) as e:
        g.append(np.array([4]), None)
    assert e.value.name == "EHOSTFULL"
    assert _same(before, g.export_state())


def test_empty_and_all_padding_steps():
    wl, tr, g = _small()
    g.step(np.zeros((0, 5), dtype=np.int64))
    assert g.last.as_tuple() == (0, 0, 0, 0, 0, 0) and g.flag == 1
    g.step(np.full((2, 3), -1))
    assert g.last.as_tuple() == (0, 0, 0, 0, 0, 6) and g.flag == 2
