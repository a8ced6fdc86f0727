"""Error paths, empty steps, ordering and determinism of the engine (GPU).

Errors found on the host return at once and change nothing; errors found on
the device are latched, the rest of the step changes nothing, ula_sync
reports them and the context refuses further work (ULA_ESTATE) while its
state stays exportable. Every error is provoked by host-chosen arguments that
the kernels check: no kernel faults or waits on purpose.
"""

import dataclasses

import numpy as np
import pytest

from digests import digest
from gpu_harness import run_parity
from oracle.replay import initial_load as oracle_load, new_group
from synth import Trace, preset, rows_for, scaled
from tracegen import tiny_workload

pytestmark = pytest.mark.gpu


def _engine(wl=None, steps=None):
    """An engine over the tiny workload with its initial history loaded."""
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device
    wl = wl or preset("tiny_4x4k")
    tr = Trace(wl, steps)
    eng = engine_for(tr, max_append=4096)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    initial_load(eng, tr, [0], rows)
    return tr, eng, rows


def _cuda(a):
    import torch
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _state(eng):
    return digest(eng.export_state(0))


@pytest.mark.parametrize("policy", [0, 1], ids=["pblru", "lru"])
@pytest.mark.parametrize("bad", ["range", "never_appended", "negative", "capacity"])
def test_device_errors_latch_and_change_nothing(bad, policy):
    from serving_pb_lru_amd import Engine, UlaError
    from synth.device import rows_device
    tr = Trace(preset("tiny_4x4k"))
    wl = tr.wl
    # max_k wide enough for a step with more distinct entries than GPU slots
    eng = Engine(1, wl.layers, wl.row_bytes, wl.ring, tr.N, tr.P, tr.H, max_sets=tr.n_sets,
                 max_k=tr.P + 1, max_append=4096, policy=policy)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    try:
        order = tr.initial_load_order()
        eng.append(0, order, rows(order, 0))
        sel = next(tr.selections(0)).copy()
        if bad == "range":
            sel[0, 5] = tr.N
        elif bad == "never_appended":
            sel[0, 5] = tr.appends(3)[0]          # reserved address, appended later
        elif bad == "negative":
            sel[0, 5] = -7
        else:
            sel = order[: tr.P + 1][None, :]       # all appended, all distinct
        want = "ECAPACITY" if bad == "capacity" else "ERANGE"
        before = _state(eng)
        d = _cuda(sel)
        eng.step(0, d)
        with pytest.raises(UlaError) as e:
            eng.sync()
        assert e.value.name == want
        assert _state(eng) == before
        for call in (lambda: eng.step(0, d), lambda: eng.gather(0, 0, d),
                     lambda: eng.gather_layers(0, 0, 1, d),
                     lambda: eng.append_step(0, tr.appends(1), rows(tr.appends(1), 0), d),
                     lambda: eng.append(0, tr.appends(1), rows(tr.appends(1), 0))):
            with pytest.raises(UlaError) as e:
                call()
            assert e.value.name == "ESTATE"
    finally:
        eng.close()


def test_host_errors_change_nothing():
    from serving_pb_lru_amd import UlaError
    tr, eng, rows = _engine()
    try:
        sel = _cuda(next(tr.selections(0)))
        with pytest.raises(UlaError) as e:
            eng.gather(0, 0, sel)                 # no step yet
        assert e.value.name == "ENOTRESIDENT"
        before = _state(eng)
        app = tr.appends(1)
        cases = [
            ("ERANGE", lambda: eng.append(0, np.array([tr.N]), rows(np.array([0]), 0))),
            ("EDUP", lambda: eng.append(0, np.array([0]), rows(np.array([0]), 0))),
            ("EDUP", lambda: eng.append(0, np.array([app[0], app[0]]), rows(np.array([0, 0]), 0))),
            ("EINVAL", lambda: eng.step(1, sel)),
            ("EINVAL", lambda: eng.step(0, _cuda(np.zeros((tr.n_sets + 1, tr.k))))),
            ("EINVAL", lambda: eng.gather(0, 1, sel)),
            # ula_append_step: a host error in either part enqueues nothing
            ("ERANGE", lambda: eng.append_step(0, np.array([tr.N]), rows(np.array([0]), 0), sel)),
            ("EDUP", lambda: eng.append_step(0, np.array([0]), rows(np.array([0]), 0), sel)),
            ("EINVAL", lambda: eng.append_step(1, app, rows(app, 0), sel)),
            ("EINVAL", lambda: eng.append_step(0, app, rows(app, 0),
                                               _cuda(np.zeros((tr.n_sets + 1, tr.k))))),
        ]
        for name, fn in cases:
            with pytest.raises(UlaError) as e:
                fn()
            assert e.value.name == name
        eng.sync()
        assert _state(eng) == before
        eng.append(0, app, rows(app, 0))   # none of the failed calls recorded these addresses
    finally:
        eng.close()


@pytest.mark.parametrize("policy", [0, 1], ids=["pblru", "lru"])
def test_append_step_device_error_keeps_the_append(policy):
    """A step that selects a never appended address fails on the device (ERANGE at
    ula_sync) and changes nothing; the append that came with it in ula_append_step
    has taken place, as it would have with ula_append before ula_step."""
    from oracle.replay import initial_load as oracle_load, new_group
    from serving_pb_lru_amd import UlaError
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device
    tr = Trace(preset("tiny_4x4k"))
    wl = tr.wl
    eng = engine_for(tr, max_append=4096, policy=policy)
    rows = lambda las: rows_device(las, wl.layers, wl.row_bytes, wl.seed, 0)
    try:
        initial_load(eng, tr, [0], lambda las, g: rows(las))
        sel = next(tr.selections(0)).copy()
        app = tr.appends(1)
        sel[0, 3] = tr.appends(2)[0]               # appended only at step 2
        eng.append_step(0, app, rows(app), _cuda(sel))
        with pytest.raises(UlaError) as e:
            eng.sync()
        assert e.value.name == "ERANGE"
        st = eng.export_state(0)
        if policy == 0:
            ora = new_group(tr, full_data=False)
            oracle_load(ora, tr, 0)
            ora.append(app, None)
            ref = ora.export_state()
            for key in ("map", "gown", "hown", "bitsets"):
                assert np.array_equal(np.asarray(st[key]), np.asarray(ref[key])), key
            assert (st["flag"], tuple(st["stats"])) == (ref["flag"], tuple(ref["stats"]))
        else:
            assert st["flag"] == 0
        assert all(st["map"][la] != 0xFFFFFFFF for la in app)
    finally:
        eng.close()


def test_gather_layers_errors():
    """ula_gather_layers: a window outside the group's layers or an empty one is
    ULA_EINVAL, no step yet is ULA_ENOTRESIDENT, an empty selection is a no-op, and
    a host-resident entry latches ULA_ENOTRESIDENT on the device as for ula_gather;
    none of them changes the state."""
    import torch
    from serving_pb_lru_amd import UlaError
    wl = dataclasses.replace(preset("tiny_4x4k"), layers=3, name="tiny_l3")
    tr, eng, rows = _engine(wl)
    try:
        sel = next(tr.selections(0))
        d = _cuda(sel)
        with pytest.raises(UlaError) as e:
            eng.gather_layers(0, 0, 3, d)         # no step yet
        assert e.value.name == "ENOTRESIDENT"
        app = tr.appends(1)
        eng.append_step(0, app, rows(app, 0), d)
        eng.sync()
        before = _state(eng)
        for l0, nl in [(-1, 1), (0, 0), (0, 4), (1, 3), (2, 2), (3, 1), (0, -1)]:
            with pytest.raises(UlaError) as e:
                eng.gather_layers(0, l0, nl, d, out=torch.empty((4, *sel.shape, wl.row_bytes),
                                                                dtype=torch.uint8, device="cuda"))
            assert e.value.name == "EINVAL", (l0, nl)
        with pytest.raises(UlaError) as e:
            eng.gather_layers(1, 0, 1, d)          # no such group
        assert e.value.name == "EINVAL"
        empty = _cuda(np.zeros((0, tr.k)))
        out = eng.gather_layers(0, 0, 3, empty)
        assert out.shape == (3, 0, tr.k, wl.row_bytes)
        eng.sync()
        assert _state(eng) == before
        st = eng.export_state(0)
        on_host = int(np.flatnonzero(st["map"] & 0x80000000 != 0)[0])
        eng.gather_layers(0, 1, 2, _cuda([[on_host]]))
        with pytest.raises(UlaError) as e:
            eng.sync()
        assert e.value.name == "ENOTRESIDENT"
        assert _state(eng) == before
    finally:
        eng.close()


def test_host_pool_full_rejected():
    from serving_pb_lru_amd import Engine, UlaError
    eng = Engine(1, 1, 64, 2, logical_capacity=16, gpu_slots=4, host_slots=4, max_sets=1, max_k=4)
    try:
        eng.append(0, np.arange(8), rows_for(0, 0, np.arange(8), 1, 64))
        before = _state(eng)
        with pytest.raises(UlaError) as e:
            eng.append(0, np.array([9]), rows_for(0, 0, [9], 1, 64))
        assert e.value.name == "EHOSTFULL"
        assert _state(eng) == before
    finally:
        eng.close()


def test_gather_of_host_resident_entry_latches():
    from serving_pb_lru_amd import UlaError
    tr, eng, rows = _engine()
    try:
        sel = next(tr.selections(0))
        app = tr.appends(1)
        eng.append(0, app, rows(app, 0))
        eng.step(0, _cuda(sel))
        eng.sync()
        st = eng.export_state(0)
        on_host = int(np.flatnonzero(st["map"] & 0x80000000 != 0)[0])
        before = digest(st)
        eng.gather(0, 0, _cuda([[on_host]]))
        with pytest.raises(UlaError) as e:
            eng.sync()
        assert e.value.name == "ENOTRESIDENT"
        assert _state(eng) == before
    finally:
        eng.close()


def test_empty_and_all_padding_steps_match_oracle():
    import torch
    tr, eng, rows = _engine()
    wl = tr.wl
    ora = new_group(tr, full_data=True)
    oracle_load(ora, tr, 0)
    try:
        for i, sel in enumerate([np.zeros((0, tr.k), np.int32), np.full((tr.n_sets, 7), -1, np.int32),
                                 next(tr.selections(0))]):
            if i == 2:   # the trace's first selection may pick the positions appended with it
                app = tr.appends(1)
                eng.append(0, app, rows(app, 0))
                ora.append(app, rows_for(wl.seed, 0, app, wl.layers, wl.row_bytes))
            d = _cuda(sel)
            eng.step(0, d)
            outs = [eng.gather(0, l, d) for l in range(wl.layers)]
            eng.sync()
            ora.step(sel)
            st = eng.export_state(0)
            ref = ora.export_state()
            assert digest(st) == digest(ref)
            for l in range(wl.layers):
                assert np.array_equal(outs[l].cpu().numpy(), ora.gather(sel, l, step=ora.flag))
    finally:
        eng.close()


def test_gather_on_second_stream_ordered_by_event():
    import torch
    tr, eng, rows = _engine()
    wl = tr.wl
    try:
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        busy = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        sel = next(tr.selections(0))
        d = _cuda(sel)
        app = tr.appends(1)
        app_rows = rows(app, 0)
        torch.cuda.synchronize()
        busy.fill_(3)                              # keeps the main stream busy for a while
        eng.append(0, app, app_rows)
        eng.step(0, d)
        done = torch.cuda.Event()
        done.record(main)
        side.wait_event(done)
        out = eng.gather(0, 0, d, stream=side)
        torch.cuda.synchronize()
        eng.sync()
        want = rows_for(wl.seed, 0, sel.reshape(-1), wl.layers, wl.row_bytes)[:, 0]
        assert np.array_equal(out.cpu().numpy().reshape(-1, wl.row_bytes), want)
    finally:
        eng.close()


def test_gather_layers_on_second_stream_and_timed():
    """Layer 0 gathered on the step's stream and the later layers by one
    ula_gather_layers launch on a second stream ordered after the step by an
    event (the prefetch of the later layers): every layer's rows match their
    closed form; with gather timing on, each launch, one layer or several,
    records one kernel duration."""
    import torch
    wl = dataclasses.replace(preset("tiny_4x4k"), layers=3, name="tiny_l3")
    tr, eng, rows = _engine(wl)
    try:
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        busy = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        eng.set_timing(eng.TIMING_GATHER)
        sels = tr.selections(0)
        for t in range(1, 4):
            sel = next(sels)
            d = _cuda(sel)
            app = tr.appends(t)
            app_rows = rows(app, 0)
            torch.cuda.synchronize()
            busy.fill_(t)                          # keeps the main stream busy for a while
            eng.append_step(0, app, app_rows, d)
            done = torch.cuda.Event()
            done.record(main)
            side.wait_event(done)
            first = eng.gather(0, 0, d)
            later = eng.gather_layers(0, 1, 2, d, stream=side)
            torch.cuda.synchronize()
            eng.sync()
            want = rows_for(wl.seed, 0, sel.reshape(-1), wl.layers, wl.row_bytes)
            assert np.array_equal(first.cpu().numpy().reshape(-1, wl.row_bytes), want[:, 0]), t
            for i in range(2):
                assert np.array_equal(later[i].cpu().numpy().reshape(-1, wl.row_bytes), want[:, 1 + i]), (t, i)
        ms, n = eng.read_gather_timing()
        assert n == 6 and ms > 0
    finally:
        eng.close()


def test_gather_on_second_stream_ordered_by_counter_wait():
    """The other ordering the boundary offers: a second stream waits on the
    group's completion counter (hipStreamWaitValue64 on ula_flag_address) until it
    reaches the step, then gathers. The first step checks, with the device idle,
    that the counter reaches its step number, so the wait of the second step
    (same kernels, valid inputs) is known to end."""
    import ctypes
    import torch
    hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch has already loaded
    hip.hipStreamWaitValue64.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                         ctypes.c_uint, ctypes.c_uint64]
    hip.hipStreamWaitValue64.restype = ctypes.c_int
    wait_gte = 0x0
    tr, eng, rows = _engine()
    wl = tr.wl
    try:
        sels = tr.selections(0)
        sel = next(sels)
        app = tr.appends(1)
        eng.append(0, app, rows(app, 0))
        eng.step(0, _cuda(sel))
        eng.sync()
        assert eng.export_state(0)["flag"] == 1
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        busy = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        sel = next(sels)
        d = _cuda(sel)
        app = tr.appends(2)
        app_rows = rows(app, 0)
        torch.cuda.synchronize()
        busy.fill_(3)                              # keeps the main stream busy for a while
        eng.append(0, app, app_rows)
        eng.step(0, d)
        rc = hip.hipStreamWaitValue64(ctypes.c_void_p(side.cuda_stream), ctypes.c_void_p(eng.flag_address(0)),
                                      2, wait_gte, 0xFFFFFFFFFFFFFFFF)
        assert rc == 0, rc
        out = eng.gather(0, 0, d, stream=side)
        torch.cuda.synchronize()
        eng.sync()
        want = rows_for(wl.seed, 0, sel.reshape(-1), wl.layers, wl.row_bytes)[:, 0]
        assert np.array_equal(out.cpu().numpy().reshape(-1, wl.row_bytes), want)
        assert eng.export_state(0)["flag"] == 2
    finally:
        eng.close()


def test_unordered_gather_is_refused_or_leaves_the_step_intact():
    """A gather issued on another stream without ordering after the step either
    finds the completion counter behind and reports ENOTRESIDENT, or runs once the
    counter has been raised. Its rows are guaranteed in neither case (ula.h: an
    unordered gather is undefined; the counter check is a relaxed read), so what
    is checked is what the design does guarantee: the gather's error never stops
    the step it raced (gather errors are latched apart from the step's status),
    so the group's state equals the oracle's after that step either way."""
    import torch
    from serving_pb_lru_amd import UlaError
    tr, eng, rows = _engine()
    wl = tr.wl
    ora = new_group(tr, full_data=False)
    oracle_load(ora, tr, 0)
    try:
        side = torch.cuda.Stream()
        busy = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        sels = tr.selections(0)
        for t in (1, 2):
            sel = next(sels)
            d = _cuda(sel)
            app = tr.appends(t)
            eng.append(0, app, rows(app, 0))
            eng.step(0, d)
            eng.sync()
            ora.append(app, None)
            ora.step(sel)
        sel = next(sels)
        d = _cuda(sel)
        app = tr.appends(3)
        app_rows = rows(app, 0)
        torch.cuda.synchronize()
        busy.fill_(1)
        eng.append(0, app, app_rows)
        eng.step(0, d)
        eng.gather(0, 0, d, stream=side)
        torch.cuda.synchronize()
        ora.append(app, None)
        ora.step(sel)
        try:
            eng.sync()
        except UlaError as e:
            assert e.name == "ENOTRESIDENT"
        st, ref = eng.export_state(0), ora.export_state()
        for key in ("map", "gown", "hown", "bitsets"):
            assert np.array_equal(st[key], ref[key]), f"{key} differs after the raced step"
        assert (st["flag"], tuple(st["stats"])) == (ref["flag"], ref["stats"])
    finally:
        eng.close()


def test_runs_are_deterministic():
    """Two runs from a fresh start must both match the oracle at every step
    (atomics may complete in any order; the state must not depend on it)."""
    wl = scaled(preset("spec3_r128_64k128k_g4"), 32)
    run_parity(wl, steps=4, groups=[0])
    run_parity(wl, steps=4, groups=[0])


def test_engine_on_dirty_workspace_matches_oracle():
    """Regression: every counter the kernels rely on is initialised by ula_init,
    whatever the workspace memory held before (here: all bits set)."""
    import torch
    from serving_pb_lru_amd import lib
    from serving_pb_lru_amd.ula import UlaConfig
    import ctypes
    wl = tiny_workload(5)
    tr = Trace(wl)
    cfg = UlaConfig(1, wl.layers, wl.row_bytes, wl.ring, tr.N, tr.P, tr.H, tr.n_sets, tr.k, 4096)
    nbytes = lib().ula_device_bytes(ctypes.byref(cfg))
    junk = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    del junk                      # the caching allocator hands this block to the engine
    run_parity(wl, max_append=4096)


def test_failed_step_marks_the_counter_and_releases_a_waiter():
    """A step that fails on the device (an address never appended) leaves the last
    completed step in the completion counter and sets bit 62, so a stream waiting
    for the counter to reach that step is released. The counter is read with the
    device idle before any wait is enqueued, so the wait is known to end; the
    gather behind it is refused and ula_sync reports the step's error."""
    import ctypes
    import torch
    hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch has already loaded
    hip.hipStreamWaitValue64.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                         ctypes.c_uint, ctypes.c_uint64]
    hip.hipStreamWaitValue64.restype = ctypes.c_int
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    wait_gte = 0x0
    tr, eng, rows = _engine()
    try:
        sels = tr.selections(0)
        sel = next(sels)
        app = tr.appends(1)
        eng.append(0, app, rows(app, 0))
        eng.step(0, _cuda(sel))
        eng.sync()
        bad = next(sels).copy()
        bad.reshape(-1)[3] = tr.N - 1            # never appended (the last step's position)
        eng.step(0, _cuda(bad))
        torch.cuda.synchronize()
        raw = ctypes.c_int64()
        assert hip.hipMemcpy(ctypes.byref(raw), ctypes.c_void_p(eng.flag_address(0)), 8, 2) == 0
        assert raw.value == (1 << 62) | 1, hex(raw.value)
        side = torch.cuda.Stream()
        rc = hip.hipStreamWaitValue64(ctypes.c_void_p(side.cuda_stream), ctypes.c_void_p(eng.flag_address(0)),
                                      2, wait_gte, 0xFFFFFFFFFFFFFFFF)
        assert rc == 0, rc
        eng.gather(0, 0, _cuda(bad), stream=side)
        torch.cuda.synchronize()
        assert eng.sync_code() == -2              # ERANGE, the step's error
        st = eng.export_state(0)
        assert st["flag"] == 1                    # exported without the failure bit
    finally:
        eng.close()


@pytest.mark.parametrize("policy", [0, 1], ids=["pblru", "lru"])
def test_timing_modes_count_and_change_nothing(policy):
    """Gather timing and link timing record one kernel duration per launch (one
    host-link launch per step); no timing mode changes any state or gathered byte."""
    from serving_pb_lru_amd import UlaError
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device
    tr = Trace(preset("tiny_4x4k"))
    wl = tr.wl
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    eng = engine_for(tr, max_append=4096, policy=policy)
    ref = engine_for(tr, max_append=4096, policy=policy)
    for e in (eng, ref):
        initial_load(e, tr, [0], rows)
    try:
        with pytest.raises(UlaError) as e:
            eng.set_timing(8)
        assert e.value.name == "EINVAL"
        eng.set_timing(eng.TIMING_STEP | eng.TIMING_GATHER | eng.TIMING_LINK)
        assert eng.read_gather_timing() == (0.0, 0)
        assert eng.read_link_timing() == (0.0, 0)
        sels = tr.selections(0)
        launches = 0
        for t in range(1, 4):
            sel = _cuda(next(sels))
            app = tr.appends(t)   # the step's selection may pick the positions appended with it
            for e in (eng, ref):
                e.append(0, app, rows(app, 0))
                e.step(0, sel)
            for l in range(tr.wl.layers):
                a, b = eng.gather(0, l, sel), ref.gather(0, l, sel)
                launches += 1
                assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())
            ms3 = eng.read_timing(0)
            assert len(ms3) == 3 and all(x >= 0 for x in ms3)
        ms, n = eng.read_gather_timing()
        assert n == launches and ms > 0
        assert eng.read_gather_timing() == (0.0, 0)   # reset by the read
        ms, n = eng.read_link_timing()
        assert n == 3 and ms > 0
        assert eng.read_link_timing() == (0.0, 0)
        eng.sync(), ref.sync()
        assert _state(eng) == _state(ref)
    finally:
        eng.close()
        ref.close()


def test_lru_empty_padding_and_dirty_workspace():
    """Exact LRU: an empty step and an all-padding step change nothing but the counter
    and statistics; an engine built on a workspace full of set bits matches the
    oracle over a whole trace (every counter and histogram the LRU kernels use is
    initialised by ula_init)."""
    import torch
    from oracle.exact_lru_np import ExactLRUArrays
    from serving_pb_lru_amd.replay import engine_for, initial_load
    from serving_pb_lru_amd import lib
    from serving_pb_lru_amd.ula import UlaConfig
    from synth.device import rows_device
    import ctypes
    wl = tiny_workload(5, steps=12)
    wl = dataclasses.replace(wl, pool_slots=2 * wl.requests * wl.sets_per_request * wl.k)
    tr = Trace(wl)
    cfg = UlaConfig(1, wl.layers, wl.row_bytes, wl.ring, tr.N, tr.P, tr.H, tr.n_sets, tr.k, 4096, 1)
    junk = torch.full((lib().ula_device_bytes(ctypes.byref(cfg)),), 0xFF, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    del junk                      # the caching allocator hands this block to the engine
    eng = engine_for(tr, max_append=4096, policy=1)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    ora = ExactLRUArrays(tr.N, tr.P, tr.H, wl.ring)
    try:
        initial_load(eng, tr, [0], rows)
        ora.append(tr.initial_load_order())
        sels = list(tr.selections(0))
        plan = [np.zeros((0, tr.k), np.int32), np.full((tr.n_sets, 5), -1, np.int32)] + sels
        t_app = 0
        for i, sel in enumerate(plan):
            if i >= 2:
                t_app += 1
                app = tr.appends(t_app)
                eng.append(0, app, rows(app, 0))
                ora.append(app)
            d = _cuda(sel)
            eng.step(0, d)
            outs = [eng.gather(0, l, d) for l in range(wl.layers)]
            eng.sync()
            ora.step(sel)
            st, ref = eng.export_state(0), ora.export_state()
            for k in ("map", "gown", "hown", "bitsets", "stamps"):
                assert np.array_equal(np.asarray(st[k]), np.asarray(ref[k])), (i, k)
            assert st["flag"] == ref["flag"] and tuple(st["stats"]) == tuple(ref["stats"]), i
            flat = sel.reshape(-1)
            want = rows_for(wl.seed, 0, np.where(flat < 0, 0, flat), wl.layers, wl.row_bytes)
            want[flat < 0] = 0
            for l in range(wl.layers):
                assert np.array_equal(outs[l].cpu().numpy().reshape(flat.size, wl.row_bytes), want[:, l])
    finally:
        eng.close()


def test_release_host_errors_change_nothing():
    from serving_pb_lru_amd import UlaError
    tr, eng, rows = _engine()
    try:
        before = _state(eng)
        first = int(tr.initial_load_order()[0])
        never = int(tr.appends(2)[0])
        for bad, name in [([tr.N], "ERANGE"), ([-3], "ERANGE"), ([never], "ERANGE"), ([first, first], "EDUP")]:
            with pytest.raises(UlaError) as e:
                eng.release(0, np.array(bad, dtype=np.int32))
            assert e.value.name == name
        assert _state(eng) == before
        # a valid release, then the same address again: not appended any more
        eng.release(0, np.array([first], dtype=np.int32))
        with pytest.raises(UlaError) as e:
            eng.release(0, np.array([first], dtype=np.int32))
        assert e.value.name == "ERANGE"
        st = eng.export_state(0)
        assert st["map"][first] == 0xFFFFFFFF
        # appended again, it takes the slot it freed (the lowest free GPU slot)
        eng.append(0, np.array([first], dtype=np.int32), rows(np.array([first], dtype=np.int32), 0))
        assert eng.export_state(0)["map"][first] == 0
        assert np.array_equal(eng.read_rows(0, np.array([first], np.int32)),
                              rows_for(tr.wl.seed, 0, np.array([first]), tr.wl.layers, tr.wl.row_bytes))
    finally:
        eng.close()
