"""ula_append_step at the edges of its one-workgroup append (GPU).

A step's appends of up to 128 entries (256 under exact LRU) run as one more
workgroup of the step's first launch; larger ones go through the
multi-workgroup append kernels before the step. Either way the result must be
exactly that of ula_append followed by ula_step: here appends of 128, 129, 256
and 257 entries per step (one request, so a step appends that many positions),
with the GPU pool full so that every appended entry takes a host slot, are
checked after every step against the oracle of each policy (state, statistics
and every gathered byte).
"""

import numpy as np
import pytest

from gpu_harness import assert_same_state, say
from oracle.exact_lru import ExactLRUGroup
from oracle.replay import initial_load as oracle_load, new_group
from synth import Trace, Workload, rows_for
from test_lru_gpu import _compare, _lru_state

pytestmark = pytest.mark.gpu


def _workload(n_app: int) -> Workload:
    return Workload(name=f"app{n_app}", requests=1, ctx_fixed=4096, ctx_range=None, sets_per_request=1,
                    draft_keep=0.5, groups=1, layers=2, k=256, pool_frac=0.0, pool_slots=2048, ring=4,
                    steps=4, appends=n_app, overlap=0.5, p_recent=0.5, window=512, row_bytes=64,
                    seed=n_app % 256)


@pytest.mark.parametrize("policy", [0, 1], ids=["pblru", "lru"])
@pytest.mark.parametrize("n_app", [128, 129, 256, 257])
def test_append_step_at_the_fused_limits(n_app, policy):
    import torch
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device
    wl = _workload(n_app)
    tr = Trace(wl)
    say(f"append limits: {n_app} appends per step, policy {policy}, N={tr.N} P={tr.P} H={tr.H}")
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    eng = engine_for(tr, max_append=1024, policy=policy)
    if policy:
        ora = ExactLRUGroup(tr.N, tr.P, tr.H)
    else:
        ora = new_group(tr, full_data=True)
    try:
        initial_load(eng, tr, [0], rows)
        if policy:
            ora.append(tr.initial_load_order())
        else:
            oracle_load(ora, tr, 0)
        sels = tr.selections(0)
        for t in range(1, tr.steps + 1):
            sel = next(sels)
            app = tr.appends(t)
            assert app.size == n_app
            dsel = torch.from_numpy(sel).cuda()
            eng.append_step(0, app, rows(app, 0), dsel)
            outs = [eng.gather(0, 0, dsel)] + list(eng.gather_layers(0, 1, 1, dsel))
            eng.sync()
            if policy:
                ora.append(app)
                ora.step(sel)
                _compare(eng.export_state(0), _lru_state(ora, tr.P), f"step {t}")
            else:
                ora.append(app, rows_for(wl.seed, 0, app, wl.layers, wl.row_bytes))
                ora.step(sel)
                assert_same_state(eng.export_state(0), ora.export_state(), f"step {t}")
            flat = sel.reshape(-1)
            want = np.zeros((flat.size, wl.layers, wl.row_bytes), np.uint8)
            ok = flat >= 0
            want[ok] = rows_for(wl.seed, 0, flat[ok], wl.layers, wl.row_bytes)
            for layer, out in enumerate(outs):
                got = out.cpu().numpy().reshape(flat.size, wl.row_bytes)
                assert np.array_equal(got, want[:, layer]), f"step {t} layer {layer}: gathered rows differ"
    finally:
        eng.close()
