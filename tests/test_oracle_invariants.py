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
