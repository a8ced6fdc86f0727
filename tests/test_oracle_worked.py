"""The oracle reproduces the hand-worked three-step example exactly.

The fixture (tests/golden/worked_example.json) is derived by hand from the
PB-LRU rules of the UlaCache summary, section 3, and states every field after
every step; exact LRU is checked on the same example (same victims).
"""

import json
import os

import numpy as np

from oracle.exact_lru import ExactLRUGroup
from oracle.invariants import check_state, check_step
from oracle.pblru import PBLRUGroup
from synth import rows_for

HERE = os.path.dirname(os.path.abspath(__file__))


def _enc(s):
    return int(s[1:]) if s[0] == "G" else (0x80000000 | int(s[1:]))


def _load():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        return json.load(f)


def test_worked_example_pblru():
    ex = _load()
    z = ex["sizes"]
    g = PBLRUGroup(z["N"], z["P"], z["H"], z["B"], z["layers"], 656, full_data=True)
    las = np.array(ex["appends"])
    g.append(las, rows_for(0, 0, las, 1, 656))
    a = ex["after_appends"]
    st = g.export_state()
    assert [int(x) for x in st["map"]] == [_enc(s) for s in a["map"]]
    assert int(st["bitsets"][0][0]) == a["free"] and int(st["bitsets"][1][0]) == a["cold"]
    assert [int(st["bitsets"][2 + b][0]) for b in range(2)] == a["ring"]
    check_state(st, z["P"], z["H"])
    for s in ex["steps"]:
        prev = g.export_state()
        g.step(np.array(s["sel"]))
        st = g.export_state()
        U, hit_slots, miss_la, miss_h, victims = g.last_lists
        assert list(U) == s["unique"]
        assert list(hit_slots) == s["hit_slots"]
        assert [[int(a), int(b)] for a, b in zip(miss_la, miss_h)] == s["misses"]
        assert list(victims) == s["victims"]
        assert [int(x) for x in st["map"]] == [_enc(x) for x in s["map"]]
        assert list(st["gown"]) == s["gown"] and list(st["hown"]) == s["hown"]
        assert int(st["bitsets"][0][0]) == s["free"]
        assert int(st["bitsets"][1][0]) == s["cold"]
        assert [int(st["bitsets"][2 + b][0]) for b in range(2)] == s["ring"]
        assert st["cur"] == s["cur"]
        assert list(st["stats"]) == s["stats"]
        check_step(prev, st, z["P"], z["H"], U=U, victims=victims, hit_slots=hit_slots)
        out = g.gather(np.array(s["sel"]), 0, step=st["flag"])
        for i, la in enumerate(s["gather"]):
            want = np.zeros(656, np.uint8) if la == -1 else rows_for(0, 0, [la], 1, 656)[0, 0]
            assert (out[0, i] == want).all()


def test_worked_example_exact_lru():
    ex = _load()
    z = ex["sizes"]
    g = ExactLRUGroup(z["N"], z["P"], z["H"])
    g.append(ex["appends"])
    for s, want in zip(ex["steps"], ex["exact_lru_victims"]):
        g.step(s["sel"])
        assert g.last_victims == want
        assert g.map_array() == [_enc(x) for x in s["map"]]


# ---- the "ring" placement of appended entries ------------------------------
def _enc2(s):
    return 0xFFFFFFFF if s == "-" else _enc(s)


def _load_ring():
    with open(os.path.join(HERE, "golden", "worked_example_ring_append.json")) as f:
        return json.load(f)


def test_worked_example_ring_append_pblru():
    """Appends into the current bucket: evictions to the lowest free host slots,
    an entry with no victim left on the host, then steps over the result; every
    field after every call, stored rows and gathered rows against their closed
    form."""
    ex = _load_ring()
    z = ex["sizes"]
    g = PBLRUGroup(z["N"], z["P"], z["H"], z["B"], z["layers"], 656, full_data=True, placement="ring")
    appended = []
    for op in ex["ops"]:
        prev = g.export_state()
        if "append" in op:
            las = np.array(op["append"])
            g.append(las, rows_for(0, 0, las, 1, 656))
            appended += op["append"]
        else:
            g.step(np.array(op["sel"]))
            assert list(g.last_lists[4]) == op["victims"]
            assert list(g.export_state()["stats"]) == op["stats"]
        st = g.export_state()
        assert [int(x) for x in st["map"]] == [_enc2(x) for x in op["map"]]
        assert list(st["gown"]) == op["gown"] and list(st["hown"]) == op["hown"]
        assert int(st["bitsets"][0][0]) == op["free"] and int(st["bitsets"][1][0]) == op["cold"]
        assert [int(st["bitsets"][2 + b][0]) for b in range(2)] == op["ring"]
        assert st["cur"] == op["cur"]
        check_state(st, z["P"], z["H"])
        if "sel" in op:
            U, hit_slots, _, _, victims = g.last_lists
            check_step(prev, st, z["P"], z["H"], U=U, victims=victims, hit_slots=hit_slots)
            out = g.gather(np.array(op["sel"]), 0, step=st["flag"])
            assert (out[0] == rows_for(0, 0, op["gather"], 1, 656)[:, 0]).all()
        for la in appended:   # every entry holds its own rows wherever it lives
            assert (g.read_row(la) == rows_for(0, 0, [la], 1, 656)[0]).all()


def test_worked_example_ring_append_exact_lru():
    ex = _load_ring()
    z = ex["sizes"]
    g = ExactLRUGroup(z["N"], z["P"], z["H"], placement="ring")
    for op in ex["ops"]:
        if "append" in op:
            g.append(op["append"])
        else:
            g.step(op["sel"])
            assert g.last_victims == op["victims"]
        assert g.map_array() == [_enc2(x) for x in op["map"]]
        assert g.gown == op["gown"] and g.hown == op["hown"]
