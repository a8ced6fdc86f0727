"""Run one trace through the HIP engine and the oracle side by side (GPU tests).

After the initial load and after every step the exported engine state (mapping
table, owners, bucket bitsets, current bucket, completion counter, step
statistics) must equal the oracle's bit for bit, and so must every gathered
byte.
"""

from __future__ import annotations

import sys

import numpy as np

from oracle.replay import initial_load as oracle_load, new_group
from serving_pb_lru_amd.replay import engine_for, initial_load
from synth import Trace, rows_for
from synth.device import rows_device

FIELDS = ("map", "gown", "hown", "bitsets")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def assert_same_state(st: dict, ref: dict, where: str) -> None:
    for key in FIELDS:
        a, b = np.asarray(st[key]), np.asarray(ref[key])
        if not np.array_equal(a, b):
            bad = np.flatnonzero(a.reshape(-1) != b.reshape(-1))
            raise AssertionError(f"{where}: {key} differs at {bad.size} places, first {bad[:5]}: "
                                 f"engine {a.reshape(-1)[bad[:5]]} oracle {b.reshape(-1)[bad[:5]]}")
    assert st["cur"] == ref["cur"], f"{where}: cur {st['cur']} vs {ref['cur']}"
    assert st["flag"] == ref["flag"], f"{where}: flag {st['flag']} vs {ref['flag']}"
    assert tuple(st["stats"]) == tuple(ref["stats"]), f"{where}: stats {st['stats']} vs {ref['stats']}"


def gather_layers_by(eng, g, layers, dsel, mode):
    """Every layer of group g's selection, as one tensor per layer, gathered by
    per-layer calls ("layer"), one call for all layers ("all"), or layer 0 alone
    and the later layers in one call ("split")."""
    if mode == "layer":
        return [eng.gather(g, l, dsel) for l in range(layers)]
    if mode == "all":
        return list(eng.gather_layers(g, 0, layers, dsel))
    assert mode == "split", mode
    outs = [eng.gather(g, 0, dsel)]
    if layers > 1:
        outs += list(eng.gather_layers(g, 1, layers - 1, dsel))
    return outs


def run_parity(wl, steps=None, selections=None, max_append=4096, groups=None, check_every=1,
               releases=None, combined=False, gather_mode="layer", placement=0):
    """selections: optional {g: list of int32 [n_sets][k]} overriding the trace's.

    The state is exported (which writes any staged evicted rows out to the host
    pool) every `check_every` steps and after the last; in between, evicted rows
    reach the host pool only through the next step's own write-back. Gathered
    rows are checked after every step. releases: optional {t: int32 addresses}
    released after step t (engine and oracle), before step t+1's appends.
    combined: each step's appends go with the step in one ula_append_step call.
    gather_mode: "layer" (one ula_gather per layer), "all" (one ula_gather_layers
    for every layer) or "split" (layer 0 alone, the later layers in one
    ula_gather_layers call).
    placement: 0 (appends into the lowest free slots) or 1 (into the current bucket).
    """
    import torch
    tr = Trace(wl, steps)
    groups = list(range(wl.groups)) if groups is None else groups
    say(f"parity {wl.name}: N={tr.N} P={tr.P} H={tr.H} groups={groups} steps={tr.steps}")
    eng = engine_for(tr, max_append=max_append, placement=placement)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    try:
        initial_load(eng, tr, groups, rows)
        ora = {}
        for g in groups:
            ora[g] = new_group(tr, full_data=True, placement="ring" if placement else "lowest")
            oracle_load(ora[g], tr, g)
            assert_same_state(eng.export_state(g), ora[g].export_state(), f"group {g} after load")
        sels = {g: (iter(selections[g]) if selections else tr.selections(g)) for g in groups}
        for t in range(1, tr.steps + 1):
            app = tr.appends(t)
            for g in groups:
                sel = next(sels[g])
                dsel = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
                if combined:
                    eng.append_step(g, app, rows(app, g), dsel)
                else:
                    if app.size:
                        eng.append(g, app, rows(app, g))
                    eng.step(g, dsel)
                outs = gather_layers_by(eng, g, wl.layers, dsel, gather_mode)
                ora[g].append(app, rows_for(wl.seed, g, app, wl.layers, wl.row_bytes))
                ora[g].step(sel)
                eng.sync()
                if t % check_every == 0 or t == tr.steps:
                    assert_same_state(eng.export_state(g), ora[g].export_state(), f"group {g} step {t}")
                for l in range(wl.layers):
                    ref = ora[g].gather(sel, l, step=t)
                    got = outs[l].cpu().numpy()
                    if not np.array_equal(got, ref):
                        bad = np.argwhere((got != ref).any(axis=-1))
                        raise AssertionError(f"group {g} step {t} layer {l}: gathered rows differ at "
                                             f"{len(bad)} rows, first {bad[:5].tolist()}")
                if releases is not None and t in releases and releases[t].size:
                    eng.release(g, releases[t])
                    ora[g].release(releases[t])
                    if t % check_every == 0:
                        assert_same_state(eng.export_state(g), ora[g].export_state(),
                                          f"group {g} after the release of step {t}")
        # stored rows of every entry, from whichever pool holds them (the host
        # pool after the last step's evicted rows are written out)
        known = np.concatenate([tr.initial_load_order()] + [tr.appends(t) for t in range(1, tr.steps + 1)])
        if releases is not None:
            gone = np.concatenate([np.zeros(0, np.int32)] + list(releases.values()))
            known = np.setdiff1d(known, gone)
        rng = np.random.default_rng([tr.N, 11])
        probe = known if known.size <= 4096 else rng.choice(known, size=4096, replace=False)
        for g in groups:
            got = eng.read_rows(g, probe)
            want = rows_for(wl.seed, g, probe, wl.layers, wl.row_bytes)
            assert np.array_equal(got, want), f"group {g}: stored rows differ after the last step"
        return ora
    finally:
        eng.close()
