"""ula_init_static: a context whose device workspace is the library's static
array (no device allocation) must behave exactly as one from ula_init.

Two contexts in a row on the same device (the second with a smaller
configuration, in the array the first one left behind) each run a trace with
every kind of call (initial load in one large append, appends of host-resident
rows, steps with their appends, gathers of every layer, a release) beside a
ula_init context driven identically; the exported state after every step and
every gathered byte must be identical, and both must equal the CPU oracle.
"""

import dataclasses

import numpy as np
import pytest

from digests import digest
from oracle.replay import initial_load as oracle_load, new_group
from synth import Trace, preset, rows_for

pytestmark = pytest.mark.gpu


def _engine(tr, static, max_append):
    from serving_pb_lru_amd import Engine
    wl = tr.wl
    return Engine(1, wl.layers, wl.row_bytes, wl.ring, tr.N, tr.P, tr.H, tr.n_sets, tr.k,
                  max_append=max_append, static_workspace=static)


def _run_pair(tr, max_append):
    import torch
    from synth.device import rows_device
    wl = tr.wl
    rows = lambda las: rows_device(las, wl.layers, wl.row_bytes, wl.seed, 0)
    ref = _engine(tr, False, max_append)
    sta = _engine(tr, True, max_append)
    ora = new_group(tr, full_data=True)
    try:
        order = tr.initial_load_order()
        for eng in (ref, sta):
            eng.append(0, order, rows(order))           # one large append (more than 128 entries)
        oracle_load(ora, tr, 0)
        assert digest(sta.export_state(0)) == digest(ref.export_state(0)) == digest(ora.export_state())
        released = set()
        sels = tr.selections(0)
        for t in range(1, tr.steps + 1):
            sel = next(sels)
            dsel = torch.from_numpy(sel).cuda()
            app = tr.appends(t)
            app_rows = rows_for(wl.seed, 0, app, wl.layers, wl.row_bytes)
            outs = {}
            for name, eng in (("ref", ref), ("static", sta)):
                if t % 2:                                  # the step's appends with the step
                    eng.append_step(0, app, rows(app), dsel)
                else:                                      # host-resident rows, then the step
                    eng.append(0, app, app_rows)
                    eng.step(0, dsel)
                outs[name] = [eng.gather(0, 0, dsel)]
                if wl.layers > 1:
                    outs[name] += list(eng.gather_layers(0, 1, wl.layers - 1, dsel))
                eng.sync()
            ora.append(app, app_rows)
            ora.step(sel)
            st_ref, st_sta = digest(ref.export_state(0)), digest(sta.export_state(0))
            assert st_sta == st_ref, f"step {t}: static-workspace state differs from ula_init's"
            assert st_ref == digest(ora.export_state()), f"step {t}: state differs from the oracle"
            for l in range(wl.layers):
                a, b = outs["static"][l].cpu().numpy(), outs["ref"][l].cpu().numpy()
                assert np.array_equal(a, b), f"step {t} layer {l}: gathered bytes differ"
                assert np.array_equal(b, ora.gather(sel, l, step=t)), f"step {t} layer {l}: vs oracle"
            if t == 3:                                     # release entries no later step selects
                later = set()
                for s in list(tr.selections(0))[3:]:
                    later |= set(int(x) for x in s.reshape(-1))
                cand = [int(x) for x in order[:200] if int(x) not in later and int(x) not in released]
                rel = np.array(cand[:40], dtype=np.int32)
                released |= set(cand[:40])
                for eng in (ref, sta):
                    eng.release(0, rel)
                ora.release(rel)
                assert digest(sta.export_state(0)) == digest(ref.export_state(0)) == \
                    digest(ora.export_state())
        probe = order[:256]
        probe = probe[~np.isin(probe, list(released))]
        assert np.array_equal(sta.read_rows(0, probe), ref.read_rows(0, probe))
    finally:
        sta.close()
        ref.close()


def test_static_workspace_equals_ula_init_on_two_calls_in_a_row():
    big = Trace(dataclasses.replace(preset("tiny_4x4k"), layers=3, name="tiny_4x4k_l3"))
    small = Trace(dataclasses.replace(preset("tiny_4x4k"), requests=2, k=128, ring=3, pool_slots=2048,
                                      name="tiny_2x4k_b3"), steps=6)
    print(f"static workspace: call 1 N={big.N} P={big.P} layers 3; call 2 N={small.N} P={small.P}",
          flush=True)
    _run_pair(big, 4096)
    _run_pair(small, 1024)


def test_static_workspace_refusals():
    """A second live context on the same device is refused (the array holds one),
    and so is a configuration larger than the array; after the first context is
    destroyed the array can be taken again."""
    from serving_pb_lru_amd import UlaError
    tr = Trace(preset("tiny_4x4k"))
    first = _engine(tr, True, 4096)
    try:
        with pytest.raises(UlaError) as e:
            _engine(tr, True, 4096)
        assert e.value.name == "EBUSY"
    finally:
        first.close()
    big = Trace(dataclasses.replace(preset("tiny_4x4k"), layers=3))
    with pytest.raises(UlaError) as e:
        _engine(big, True, 1 << 16)   # 144 MiB of workspace
    assert e.value.name == "ETOOBIG"
    again = _engine(tr, True, 4096)
    again.close()
