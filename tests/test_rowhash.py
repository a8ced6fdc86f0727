"""Row contents: splitmix64 and the row formula (synthetic inputs).

The splitmix64 sequence seeded with 1234567 is a widely published test vector
of the generator of Steele, Lea and Flood as given by Vigna; the row formula
packs (seed, group, layer, address, word) into disjoint bit fields.
"""

import numpy as np

from synth import row, rows_for, splitmix64

GOLDEN = 0x9E3779B97F4A7C15


def test_splitmix64_published_sequence():
    state = 1234567
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    got = []
    for _ in range(5):
        got.append(int(splitmix64(np.array([state], dtype=np.uint64))[0]))
        state = (state + GOLDEN) % 2 ** 64
    assert got == want


def test_row_fields_are_disjoint_and_rows_differ():
    a = row(0, 0, 5, 0, 656)
    assert a.size == 656 and a.dtype == np.uint8
    others = [row(1, 0, 5, 0, 656), row(0, 1, 5, 0, 656), row(0, 0, 5, 1, 656), row(0, 0, 6, 0, 656)]
    for o in others:
        assert not np.array_equal(a, o)
    x = (5 << 7) ^ np.arange(82, dtype=np.uint64)
    assert np.array_equal(a.view("<u8"), splitmix64(x))
    x = np.uint64((3 << 56) ^ (7 << 47) ^ (2 << 39) ^ ((2 ** 31 - 1) << 7) ^ 81)
    assert row(3, 7, 2 ** 31 - 1, 2, 656).view("<u8")[81] == splitmix64(np.array([x]))[0]


def test_rows_for_matches_row():
    las = np.array([0, 1, 17, 123456, 2 ** 31 - 1])
    r = rows_for(2, 3, las, 3, 656, chunk=2)
    for i, la in enumerate(las):
        for layer in range(3):
            assert np.array_equal(r[i, layer], row(2, 3, int(la), layer, 656))
