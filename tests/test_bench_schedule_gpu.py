"""Full-size parity in bench.py's timed launch configuration.

Every group of the workload runs in one engine, as in bench.py: each step's
appends and the step go in one ula_append_step call on the step stream bench.py
uses for that number of groups (one stream for one group, a stream per group for
two, two streams with the groups alternating for more), and every gather goes
to a separate gather stream after an event its step recorded (layer 0 alone, the
later layers of a group in one ula_gather_layers launch). Nothing else orders
the calls: the library makes each group's next swap wait for that group's
gathers. There is no host synchronisation until the last step. Then every
gathered byte of every step and layer must equal its closed form (rows made on
the device by synth's generator, zeros for padding), and each group's final
state digest and statistics must equal those the CPU oracle produced
(tests/golden/digests_<workload>.json).
"""

import numpy as np
import pytest

from digests import digest
from gpu_harness import say
from synth import Trace, preset
from test_parity_full_gpu import _cmp, _golden

pytestmark = pytest.mark.gpu


def _streams(torch, groups):
    if groups == 1:
        return [torch.cuda.Stream()]
    if groups == 2:
        return [torch.cuda.Stream(), torch.cuda.Stream()]
    pair = [torch.cuda.Stream(), torch.cuda.Stream()]
    return [pair[g % 2] for g in range(groups)]


def run_scheduled(name, groups=None, steps=None):
    import dataclasses

    import torch
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device

    wl = preset(name)
    if groups:
        wl = dataclasses.replace(wl, groups=groups)
    tr = Trace(wl, steps)
    G, L = wl.groups, wl.layers
    gold = _golden(name)["groups"]
    say(f"bench schedule {name}: groups={G} layers={L} steps={tr.steps} N={tr.N} P={tr.P} H={tr.H}")
    torch.cuda.set_device(0)
    main = torch.cuda.current_stream()
    rows = lambda las, g: rows_device(las, L, wl.row_bytes, wl.seed, g)
    eng = engine_for(tr, max_append=1 << 16)
    try:
        initial_load(eng, tr, range(G), rows)
        sels = {g: list(tr.selections(g)) for g in range(G)}
        dsel = {g: [torch.from_numpy(s).cuda() for s in sels[g]] for g in range(G)}
        app_rows = {(g, t): rows(tr.appends(t), g) for g in range(G) for t in range(1, tr.steps + 1)}
        outs = {(g, t): torch.empty((L, tr.n_sets, tr.k, wl.row_bytes), dtype=torch.uint8, device="cuda")
                for g in range(G) for t in range(1, tr.steps + 1)}
        torch.cuda.synchronize()
        step_s = _streams(torch, G)
        gather_s = torch.cuda.Stream()
        done = [torch.cuda.Event() for _ in range(G)]
        for t in range(1, tr.steps + 1):
            for g in range(G):
                s = step_s[g]
                eng.append_step(g, tr.appends(t), app_rows[(g, t)], dsel[g][t - 1], stream=s)
                done[g].record(s)
                gather_s.wait_event(done[g])
                o = outs[(g, t)]
                eng.gather(g, 0, dsel[g][t - 1], out=o[0], stream=gather_s)
                if L > 1:
                    eng.gather_layers(g, 1, L - 1, dsel[g][t - 1], out=o[1:], stream=gather_s)
        torch.cuda.synchronize()
        stats = eng.sync(stream=main)
        for g in range(G):
            for t in range(1, tr.steps + 1):
                sel = dsel[g][t - 1].reshape(-1)
                want = rows(sels[g][t - 1].reshape(-1), g)
                want[sel == -1] = 0
                for l in range(L):
                    got = outs[(g, t)][l].reshape(-1, wl.row_bytes)
                    if not torch.equal(got, want[:, l]):
                        bad = (got != want[:, l]).any(dim=1).nonzero().reshape(-1)[:5].tolist()
                        raise AssertionError(f"{name} g{g} step {t} layer {l}: gathered rows differ, "
                                             f"first rows {bad}")
                del want
            T = tr.steps
            assert list(stats[g]) == gold[g][T]["stats"], f"{name} g{g}: ula_sync stats {stats[g]}"
            _cmp(digest(eng.export_state(g)), gold[g][T], f"{name} g{g} after step {T}")
    finally:
        eng.close()


@pytest.mark.parametrize("name,groups", [("r16_64k_g1x3", None), ("evict_r256_128k_g2", None),
                                         ("spec3_r128_64k128k_g4", None), ("r64_64k128k_g24x3", 4)])
def test_bench_schedule_full_size(name, groups):
    run_scheduled(name, groups)
