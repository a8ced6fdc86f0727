"""Logical addresses at the top of the 31-bit range (GPU).

The largest logical capacity the ABI takes is N = 2^31 - 1, so the engine's
mapping and de-duplication tables hold 2^31 - 1 entries (8.6 GB and 17.2 GB of
HBM) and addresses reach 2^31 - 2. Nothing in the method depends on the values
of the addresses: de-duplication keeps first occurrences in selection order and
every other rule works on slots (UlaCache summary, sections 2 and 3). So a trace
whose addresses are relabelled by an injective map f must leave the bucket
bitsets, the counters and the statistics unchanged and relabel the mapping
table and the owners by f; the oracle's own metamorphic tests pin that property
(tests/test_oracle_metamorphic.py).

Here the oracle runs a small trace on compact addresses [0, n) and the engine the
same trace with every address a sent to f(a): a third of them the highest
addresses of the range, a sixth the lowest, the rest spread between, in shuffled
order. After the load and after every step the engine's state must equal the
oracle's relabelled one (the whole 2^31 - 1-entry mapping table: f's entries
equal, every other entry absent), and every gathered byte and every stored row
must equal the closed-form row of its relabelled address.
"""

import numpy as np
import pytest

from gpu_harness import say
from oracle.pblru import ABSENT
from oracle.replay import initial_load as oracle_load, new_group
from synth import Trace, Workload, rows_for

pytestmark = pytest.mark.gpu

N_MAX = 2 ** 31 - 1


def _relabel(n: int, seed: int) -> np.ndarray:
    """An injective map [0, n) -> [0, N_MAX) that takes the top and bottom of the range."""
    rng = np.random.default_rng([seed, 31])
    n_top, n_low = n // 3, n // 6
    top = N_MAX - 1 - np.arange(n_top, dtype=np.int64)            # N_MAX - 1 = 2^31 - 2 first
    low = np.arange(n_low, dtype=np.int64)
    mid = np.unique(rng.integers(n_low, N_MAX - n_top, size=4 * n))
    mid = rng.permutation(mid)[: n - n_top - n_low]
    f = np.concatenate([top, low, mid])
    assert f.size == n and np.unique(f).size == n
    return rng.permutation(f)


def _check(eng, ora, f, where):
    st, ref = eng.export_state(0), ora.export_state()
    assert np.array_equal(st["bitsets"], ref["bitsets"]), f"{where}: bitsets"
    assert (st["cur"], st["flag"]) == (ref["cur"], ref["flag"]), f"{where}: cur/flag"
    assert tuple(st["stats"]) == tuple(ref["stats"]), f"{where}: stats {st['stats']} vs {ref['stats']}"
    for key in ("gown", "hown"):
        want = np.where(ref[key] >= 0, f[np.maximum(ref[key], 0)], -1)
        assert np.array_equal(st[key].astype(np.int64), want), f"{where}: {key}"
    m = st["map"]
    assert m.size == N_MAX
    assert np.array_equal(m[f], ref["map"]), f"{where}: map at the relabelled addresses"
    assert np.count_nonzero(m != ABSENT) == np.count_nonzero(ref["map"] != ABSENT), \
        f"{where}: map entries outside the relabelled addresses"


@pytest.mark.parametrize("combined", [False, True], ids=["append_then_step", "append_step"])
def test_top_of_address_range(combined):
    import torch
    from serving_pb_lru_amd import Engine
    from synth.device import rows_device
    wl = Workload(name="top31", requests=4, ctx_fixed=700, ctx_range=None, sets_per_request=1,
                  draft_keep=0.5, groups=1, layers=2, k=160, pool_frac=0.0, pool_slots=1100,
                  ring=4, steps=10, appends=2, overlap=0.7, p_recent=0.5, window=64,
                  row_bytes=64, seed=9)
    tr = Trace(wl)
    f = _relabel(tr.N, seed=int(combined))
    rows = lambda las: rows_device(f[las].astype(np.int32), wl.layers, wl.row_bytes, wl.seed, 0)
    say(f"top of range: N={N_MAX} (oracle {tr.N}) P={tr.P} H={tr.H} steps={tr.steps} "
        f"highest address {f.max()}")
    eng = Engine(1, wl.layers, wl.row_bytes, wl.ring, N_MAX, tr.P, tr.H, tr.n_sets, tr.k,
                 max_append=512)
    ora = new_group(tr, full_data=False)
    try:
        order = tr.initial_load_order()
        eng.append(0, f[order].astype(np.int32), rows(order))
        oracle_load(ora, tr, 0)
        _check(eng, ora, f, "after load")
        sels = tr.selections(0)
        pad = np.random.default_rng([wl.seed, 5])
        for t in range(1, tr.steps + 1):
            sel = next(sels).copy()
            sel[pad.random(sel.shape) < 0.05] = -1
            sel[:, -3:] = sel[:, :3]                      # repeated entries in every set
            gsel = np.where(sel >= 0, f[np.maximum(sel, 0)], -1).astype(np.int32)
            dsel = torch.from_numpy(gsel).cuda()
            app = tr.appends(t)
            if combined:
                eng.append_step(0, f[app].astype(np.int32), rows(app), dsel)
            else:
                eng.append(0, f[app].astype(np.int32), rows(app))
                eng.step(0, dsel)
            ora.append(app, None)
            ora.step(sel)
            outs = [eng.gather(0, 0, dsel)] + list(eng.gather_layers(0, 1, 1, dsel))
            stats = eng.sync()[0]
            assert tuple(stats) == ora.last.as_tuple(), f"step {t}: stats"
            valid = gsel >= 0
            for layer, out in enumerate(outs):
                got = out.cpu().numpy()
                want = np.zeros_like(got)
                want[valid] = rows_for(wl.seed, 0, gsel[valid], wl.layers, wl.row_bytes)[:, layer]
                assert np.array_equal(got, want), f"step {t}: gathered bytes of layer {layer}"
            if t in (1, tr.steps // 2, tr.steps):
                _check(eng, ora, f, f"step {t}")
                say(f"  step {t}: state equal ({stats})")
        # stored rows of host- and GPU-resident entries, the highest addresses included
        alive = np.flatnonzero(ora.map != ABSENT)
        pick = np.concatenate([alive[np.argsort(f[alive])[-64:]], alive[:64]])
        got = eng.read_rows(0, f[pick].astype(np.int32))
        assert np.array_equal(got, rows_for(wl.seed, 0, f[pick], wl.layers, wl.row_bytes))
    finally:
        eng.close()
