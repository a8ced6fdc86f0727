"""Measurement probes with the plain row moves of libprobes.so.

link(): the miss path's traffic with nothing else in the launch: `rows` random
host-pool rows read into contiguous HBM (zero-copy loads of pinned host memory) and
as many contiguous HBM rows written to other random host slots, alone and both at
once on two streams, over several launch shapes; beside them a contiguous copy-engine
transfer of the same bytes (hipMemcpyAsync: alone each way, both ways at once, and
device to host beside the zero-copy reads).

gather(): `rows` random slots of an HBM pool read into a contiguous buffer, with
plain and with non-temporal loads, each launch right behind a 1 GiB write that pushes
the pool out of the memory-side cache (cold), or right behind the same gather (warm).

copy(): a contiguous device copy of the same bytes as a gather of `rows` rows (no
row indexing at all), with plain and with non-temporal loads, each launch right behind
another copy, over several launch shapes and beside torch's own copy: the HBM rate a
launch of that size reaches.

Times are per launch (events on the launch's stream, median of `reps`), each timed
launch enqueued behind other work on its stream (link(): a 256 MiB device fill), so
that the host's launch time stays out of the interval; the row indexes are checked
once, before the timed launches.
"""

import ctypes
import os
import statistics

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprobes.so")
_lib = None

LINK_PEAK_GBPS = 63.0     # PCIe 5.0 x16 per direction: 32 GT/s x 16 x 128/130 / 8
HBM_PEAK_GBPS = 8000.0


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with measure.build.build()")
        # torch ships its own HIP runtime under the same soname as the one this
        # library links; importing torch first makes the library bind to that
        # runtime (loaded the other way round, the process ends up with two HIP
        # runtimes and device calls fail)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.probe_move_rows.restype = ctypes.c_int
        L.probe_move_rows.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_uint64]
        L.probe_copy.restype = ctypes.c_int
        L.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_uint64]
        _lib = L
    return _lib


def check_move(mode: int, src, idx, dst, n: int, row_bytes: int) -> None:
    """Every index of a row move must be a row of the buffer it indexes, and the
    contiguous side must hold n rows: checked on the host (with a device sync)."""
    import torch
    assert mode in (0, 1, 2)
    assert idx.dtype == torch.int32 and idx.is_cuda and idx.numel() >= n
    indexed = src if mode != 1 else dst
    other = dst if mode != 1 else src
    if n:
        hi = int(idx[:n].max().item())
        lo = int(idx[:n].min().item())
        assert 0 <= lo and (hi + 1) * row_bytes <= indexed.numel(), "row index outside its buffer"
    assert n * row_bytes <= other.numel()


def move_rows(mode: int, src, idx, dst, n: int, row_bytes: int, blocks: int, stream,
              checked: bool = False) -> None:
    """mode 0: dst row r = src row idx[r]; mode 1: dst row idx[r] = src row r (r < n);
    mode 2: as mode 0 with non-temporal loads.
    Every index must be a row of the buffer it indexes: checked here before the launch,
    unless the caller has run check_move on the same arguments (checked=True), as the
    timed loops do so that the check's sync stays out of the timed interval."""
    if not checked:
        check_move(mode, src, idx, dst, n, row_bytes)
    rc = lib().probe_move_rows(mode, src.data_ptr(), idx.data_ptr(), dst.data_ptr(), n, row_bytes, blocks,
                               stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"probe_move_rows failed ({rc})")


def copy_bytes(src, dst, nbytes: int, blocks: int, stream, nt: bool = False) -> None:
    """dst[:nbytes] = src[:nbytes] (device tensors, checked here before the launch);
    nt: non-temporal loads."""
    assert src.is_cuda and dst.is_cuda
    assert nbytes <= src.numel() * src.element_size() and nbytes <= dst.numel() * dst.element_size()
    rc = lib().probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks, int(nt), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"probe_copy failed ({rc})")


def _timed(first, second, s1, s2, reps, lead):
    """Median over reps of the time from a start event on s1 to the later of the two
    streams' end events (second may be None). lead(s1) is enqueued on s1 right before
    the start event, so that the stream is still busy while the host enqueues the
    timed launches (on an idle stream the start event fires at once and the host's
    launch time falls into the interval)."""
    import torch
    out = []
    for _ in range(reps + 1):          # the first round warms up and is dropped
        torch.cuda.synchronize()
        lead(s1)
        st = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e2 = torch.cuda.Event(enable_timing=True)
        st.record(s1)
        s2.wait_event(st)
        first(s1)
        e1.record(s1)
        if second:
            second(s2)
        e2.record(s2)
        torch.cuda.synchronize()
        out.append(max(st.elapsed_time(e1), st.elapsed_time(e2)))
    return statistics.median(out[1:])


def link(rows: int, slot_bytes: int, host_rows: int, shapes=(96, 256, 1024), reps: int = 5,
         seed: int = 1) -> dict:
    import numpy as np
    import torch
    assert 2 * rows <= host_rows
    torch.cuda.set_device(0)
    host = torch.empty(host_rows * slot_bytes, dtype=torch.uint8, pin_memory=True)
    contig = torch.empty(rows * slot_bytes, dtype=torch.uint8, pin_memory=True)
    contig2 = torch.empty(rows * slot_bytes, dtype=torch.uint8, pin_memory=True)
    perm = np.random.default_rng(seed).permutation(host_rows)[:2 * rows].astype(np.int32)
    rd_idx = torch.from_numpy(perm[:rows].copy()).cuda()
    wr_idx = torch.from_numpy(perm[rows:].copy()).cuda()
    dev_in = torch.empty(rows * slot_bytes, dtype=torch.uint8, device="cuda")
    dev_out = torch.randint(0, 256, (rows * slot_bytes,), dtype=torch.uint8, device="cuda")
    busy = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    check_move(0, host, rd_idx, dev_in, rows, slot_bytes)
    check_move(1, dev_out, wr_idx, host, rows, slot_bytes)

    def lead(s):
        with torch.cuda.stream(s):
            busy.fill_(1)

    def rd(b):
        return lambda s: move_rows(0, host, rd_idx, dev_in, rows, slot_bytes, b, s, checked=True)

    def wr(b):
        return lambda s: move_rows(1, dev_out, wr_idx, host, rows, slot_bytes, b, s, checked=True)

    def d2h(s):
        with torch.cuda.stream(s):
            contig.copy_(dev_out, non_blocking=True)

    def h2d(s):
        with torch.cuda.stream(s):
            dev_in.copy_(contig2, non_blocking=True)

    ms = {}
    for b in shapes:
        ms[f"read_{b}"] = _timed(rd(b), None, s1, s2, reps, lead=lead)
        ms[f"write_{b}"] = _timed(wr(b), None, s1, s2, reps, lead=lead)
        ms[f"both_{b}"] = _timed(rd(b), wr(b), s1, s2, reps, lead=lead)
        ms[f"read_{b}+copy_d2h"] = _timed(rd(b), d2h, s1, s2, reps, lead=lead)
    ms["copy_d2h"] = _timed(d2h, None, s1, s2, reps, lead=lead)
    ms["copy_h2d"] = _timed(h2d, None, s1, s2, reps, lead=lead)
    ms["copy_both"] = _timed(h2d, d2h, s1, s2, reps, lead=lead)
    mb = rows * slot_bytes / 1e6
    best = min((v, k) for k, v in ms.items() if k.startswith("both_"))
    return {"rows": rows, "slot_bytes": slot_bytes, "host_rows": host_rows, "MB_each_way": round(mb, 3),
            "ms": {k: round(v, 4) for k, v in ms.items()},
            "both_best": {"shape": best[1], "ms": round(best[0], 4),
                          "GBps_each_way": round(mb / best[0], 2),
                          "frac_of_peak": round(mb / best[0] / LINK_PEAK_GBPS, 4)}}


def gather(rows: int, slot_bytes: int, pool_rows: int, shapes=(1024, 4096, 16384), reps: int = 7,
           seed: int = 2) -> dict:
    import numpy as np
    import torch
    assert rows <= pool_rows
    torch.cuda.set_device(0)
    pool = torch.randint(0, 256, (pool_rows * slot_bytes,), dtype=torch.uint8, device="cuda")
    idx = torch.from_numpy(np.random.default_rng(seed).permutation(pool_rows)[:rows].astype(np.int32)).cuda()
    out = torch.empty(rows * slot_bytes, dtype=torch.uint8, device="cuda")
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    check_move(0, pool, idx, out, rows, slot_bytes)
    state = {"i": 0}

    def evict_caches(s):
        state["i"] += 1
        with torch.cuda.stream(s):
            flush.fill_(state["i"] & 0xFF)

    def run(b, mode):
        return lambda s: move_rows(mode, pool, idx, out, rows, slot_bytes, b, s, checked=True)

    ms = {}
    for mode, tag in ((0, ""), (2, "_nt")):
        for b in shapes:
            ms[f"gather{tag}_{b}"] = _timed(run(b, mode), None, s1, s2, reps, lead=evict_caches)
            ms[f"gather{tag}_{b}_warm"] = _timed(run(b, mode), None, s1, s2, reps, lead=run(b, mode))
    algo = 2 * rows * slot_bytes
    best = min((v, k) for k, v in ms.items() if not k.endswith("_warm"))
    return {"rows": rows, "slot_bytes": slot_bytes, "pool_rows": pool_rows, "algorithmic_MB": round(algo / 1e6, 3),
            "ms": {k: round(v, 4) for k, v in ms.items()},
            "cold_best": {"shape": best[1], "us": round(best[0] * 1e3, 2),
                          "GBps": round(algo / best[0] / 1e6, 1),
                          "frac_of_peak": round(algo / best[0] / 1e6 / HBM_PEAK_GBPS, 4)}}


def copy(rows_list, slot_bytes: int, shapes=(1024, 4096, 16384, 0), reps: int = 7) -> dict:
    """Per size: a contiguous copy of rows x slot_bytes bytes (the algorithmic bytes of
    a gather of that many rows: as many read as written), each launch right behind
    another copy (of the same size, at least 256 MiB) on its stream, between other
    buffers (as a gather runs in a step loop: its source is not in the caches, which
    hold the previous launch's written lines). Shape 0 = one round per lane (as many
    workgroups as the pieces need)."""
    import torch
    torch.cuda.set_device(0)
    lead_min = 256 << 20      # long enough that the host has enqueued the timed launch
    most = max(max(rows_list) * slot_bytes, lead_min)
    src = torch.randint(0, 256, (2, most), dtype=torch.uint8, device="cuda")
    dst = torch.empty((2, most), dtype=torch.uint8, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

    def lead(nb):
        nb = max(nb, lead_min)
        def run(s):
            copy_bytes(src[0], dst[0], nb, -(-nb // (16 * 256 * 4)), s)
        return run

    def torch_copy(nb):
        def run(s):
            with torch.cuda.stream(s):
                dst[1, :nb].copy_(src[1, :nb])
        return run

    sizes = []
    for rows in rows_list:
        nb = rows * slot_bytes
        ms = {}
        for nt in (False, True):
            for b in shapes:
                blocks = b or -(-nb // (16 * 256 * 4))
                ms[f"copy{'_nt' if nt else ''}_{b or 'one_round'}"] = _timed(
                    lambda s: copy_bytes(src[1], dst[1], nb, blocks, s, nt=nt), None, s1, s2, reps, lead=lead(nb))
        ms["torch_copy"] = _timed(torch_copy(nb), None, s1, s2, reps, lead=lead(nb))
        for nt in (False, True):
            dst[1, :nb].zero_()
            copy_bytes(src[1], dst[1], nb, shapes[0] or 1024, torch.cuda.current_stream(), nt=nt)
            torch.cuda.synchronize()
            assert torch.equal(dst[1, :nb], src[1, :nb]), "probe_copy moved the wrong bytes"
        algo = 2 * nb
        best = min((v, k) for k, v in ms.items() if k != "torch_copy")
        sizes.append({"rows": rows, "algorithmic_MB": round(algo / 1e6, 3),
                      "us": {k: round(v * 1e3, 2) for k, v in ms.items()},
                      "best": {"shape": best[1], "us": round(best[0] * 1e3, 2),
                               "GBps": round(algo / best[0] / 1e6, 1),
                               "frac_of_peak": round(algo / best[0] / 1e6 / HBM_PEAK_GBPS, 4)}})
    return {"slot_bytes": slot_bytes, "sizes": sizes}
