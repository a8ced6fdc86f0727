#!/usr/bin/env python3
"""Throughput of the PB-LRU KV residency engine on one MI355X.

One step = the whole per-decode-step path for every layer group of the
workload: the step's appends and the step in one ula_append_step call (the
appends, de-duplication and lookup, fold and hit marking, victim selection, the
miss path over the host link, commit and completion signal), then the gather
of the group's first layer (ula_gather) and of its later layers in one
ula_gather_layers launch (the layers of a group share the selection, and the
later ones are fetched together while the first is in use; --gather layer
gathers each layer by its own ula_gather call, --gather all every layer in one
launch). Inputs (selection sets for every step
and the appended rows) are resident in HBM before the timed region; the GPU
pool starts full (initial load untimed). W warm-up steps run first (they carry
the cold-start misses), then exactly K steps are timed between two device
synchronisations.

value = selected row-layers resolved and gathered per second
      = K * sum over groups of (n_sets * k * layers) / timed wall seconds.

Printed as one JSON line, with:
  roofline      the step's dominant kernel against its peak. On a workload
                whose step moves rows over the host link for longer than it
                gathers (the default one) that is the host-link launch k_mark:
                the larger direction's algorithmic bytes per launch (656 x
                layers per missed row in, per evicted row of the previous step
                out; both directions move at once) over its average duration,
                from HIP events the launch records in its own dispatch (in one
                more replay of the same timed steps: the replays that give the
                value carry no such events), against 63 GB/s per direction;
                `traffic` is the counted host-link bytes of rocprofv3's IO
                request counters where they were taken for the same k_mark
                code. Otherwise the gather (below).
  roofline_other the other one: the gather against HBM peak (1312 algorithmic
                bytes per gathered row-layer: 656 read + 656 written), its
                average duration alone (the per-phase replay runs each group's
                gathers right behind its step with nothing beside them), with
                its duration inside the timed steps next to it;
  replays       the value of each of the three timed replays (value = median);
                instrumented_ms_per_step is the step time of the replay that
                carries the kernels' timing events;
  miss_path     the per-phase replay: phase times per group step, GPU hit
                rate, and hipMemcpyAsync pinned-host peaks (each direction and
                both at once) next to the host-link rates;
  cpu_baseline  the CPU oracle timed on this host's cores over the same steps
                (a bounded sample; a baseline, not the target).
Also: selections_per_s (selection entries resolved per second, all groups),
first_step_ms (step 1, the cold start with the most misses, timed alone, after
every step kernel has run once on a tiny engine) and host_enqueue_ms_per_step (the
host's time to enqueue a timed step's calls, median replay, including any wait of
an append of more than 128 entries (256 under exact LRU) for a staging buffer: near
ms_per_step with no
such appends, the GPU waits for the host).

Other modes print their own line and exit: --layer-prefetch (the later-layer
prefetch experiment), --copy-ceiling and --calibrate-copy (plain device copies:
the HBM rate at the gather's sizes, the counter scale), --link-probe and
--gather-probe (plain moves of random rows, one direction per launch, and
copy-engine transfers of the same bytes, measure/libprobes.so: the simple and
the alternative forms of the miss path's and the gather's traffic), --copy-probe
(a contiguous device copy of a gather's bytes by launch size, the same library).
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, "1")

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from synth import Trace, preset  # noqa: E402

METRIC = "selected KV rows resolved+gathered/s; gather GB/s and miss GB/s vs peak"
HBM_PEAK_GBS = 8000.0                    # MI355X HBM3E
LINK_PEAK_GBS = 32 * 16 * 128 / 130 / 8  # PCIe 5.0 x16 per direction = 63.0 GB/s
DEFAULT_WORKLOAD = "evict_r256_128k_g2"


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=14)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--replays", type=int, default=3, help="timed replays from a fresh start (median reported)")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="timed CPU work of the oracle sample (three single-core replays)")
    p.add_argument("--no-cpu-parallel", action="store_true", help="skip the groups-in-parallel CPU figure")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-phases", action="store_true", help="skip the per-phase replay")
    p.add_argument("--groups", type=int, default=0,
                   help="run only the first N layer groups of the workload (groups are independent; "
                        "for workloads whose pinned host pools exceed one host's memory)")
    p.add_argument("--first-group", type=int, default=0, metavar="G0",
                   help="with --groups N: run groups G0..G0+N-1 of the workload instead of the first N "
                        "(the same traces as in the full workload; no CPU baseline, no counters)")
    p.add_argument("--policy", choices=("pblru", "lru"), default="pblru",
                   help="replacement policy: PB-LRU (the pages' policy) or exact LRU (the one it is "
                        "compared against); the CPU baseline is reported for PB-LRU only")
    p.add_argument("--placement", choices=("lowest", "ring"), default="lowest",
                   help="where appended entries go: the lowest free slot, GPU first, never evicting "
                        "(default), or the current bucket, evicting (PB-LRU only)")
    p.add_argument("--streams", choices=("auto", "one", "group", "two", "one+gather", "group+gather",
                                         "two+gather"), default="auto",
                   help="where each group's calls go. one: one stream for every call; group: a "
                        "stream per group (one group's HBM phases run beside another's host-link "
                        "launch; the library keeps the host-link launches one at a time); two: two "
                        "streams with the groups alternating over them; X+gather: the steps as in X "
                        "and every gather on a stream of its own, after an event its step recorded "
                        "(the library makes the group's next row moves wait for it, so the next "
                        "step's lookup and marking run beside it). auto (default): one+gather for one "
                        "group, group+gather for two, two+gather for more (HIP spreads a process's "
                        "streams over four hardware queues, two of them left for created streams, "
                        "and a queue runs its launches in order); without the gather stream under "
                        "--placement ring")
    p.add_argument("--gather", choices=("layer", "split", "all"), default="split",
                   help="gathers per group step: one per layer (ula_gather); layer 0 alone, then the "
                        "later layers in one ula_gather_layers launch (default); or every layer in "
                        "one launch")
    p.add_argument("--layer-prefetch", type=float, default=0.0, metavar="US",
                   help="only run the later-layer prefetch experiment with US microseconds of "
                        "synthetic compute per layer, and print its own JSON line")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run 5 plain device-to-device copies of MIB MiB (counter calibration) and exit")
    p.add_argument("--copy-ceiling", type=int, default=0, metavar="BYTES",
                   help="only run plain device-to-device copies moving BYTES each (half read, half "
                        "written), from buffers larger than the memory-side cache, and exit")
    p.add_argument("--link-probe", type=int, default=0, metavar="ROWS",
                   help="only time plain moves of ROWS random host-pool rows into HBM and as many out "
                        "to other random host slots (each alone, both at once, and next to copy-engine "
                        "transfers) with measure/libprobes.so, print one JSON line and exit")
    p.add_argument("--gather-probe", type=int, default=0, metavar="ROWS",
                   help="only time a plain gather of ROWS random HBM-pool slots into a contiguous "
                        "buffer with measure/libprobes.so, cold and warm, print one JSON line and exit")
    p.add_argument("--copy-probe", type=str, default="", metavar="ROWS[,ROWS...]",
                   help="only time a contiguous device copy of ROWS x --slot-bytes bytes (a gather's "
                        "algorithmic bytes with no row indexing) with measure/libprobes.so, each launch "
                        "behind another copy, over several launch shapes and beside torch's copy, print "
                        "one JSON line and exit")
    p.add_argument("--slot-bytes", type=int, default=656, help="row size of the probes")
    p.add_argument("--pool-rows", type=int, default=0,
                   help="rows of the probe's pool (host pool for --link-probe, HBM pool for "
                        "--gather-probe)")
    return p.parse_args()


def calibrate_copy(mib: int) -> None:
    """A plain copy of known size, so that HBM byte counters can be scaled."""
    import torch
    torch.cuda.set_device(0)
    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": mib << 20, "copies": 5}), flush=True)


def copy_ceiling(nbytes: int, copies: int = 64) -> None:
    """Plain device-to-device copies moving `nbytes` per copy (half read, half
    written: the algorithmic bytes of one gather launch), rotating over slices
    of buffers larger than the memory-side cache so that every copy reads from
    HBM, as the gathers do. Run under rocprofv3 --kernel-trace --stats for the
    copy kernel's duration: the practical HBM rate at the gather's size."""
    import torch
    torch.cuda.set_device(0)
    half = nbytes // 2
    slices = max(4, -(-(1 << 30) // half))   # more than 1 GiB in each buffer
    src = torch.empty(slices * half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.fill_(0)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(copies):
        j = (i % slices) * half
        dst[j:j + half].copy_(src[j:j + half])
    b.record()
    torch.cuda.synchronize()
    print(json.dumps({"copy_ceiling_bytes_per_copy": 2 * half, "copies": copies, "slices": slices,
                      "batch_ms_per_copy_incl_launch_gaps": round(a.elapsed_time(b) / copies, 5)}),
          flush=True)


def schedule_for(groups: int, placement: str, streams: str = "auto") -> str:
    """The stream schedule of --streams auto (measured fastest, or as fast, on each
    workload): the steps on one stream for one group, a stream per group for two,
    two alternating streams for more (HIP spreads a process's streams over four
    hardware queues, and a queue runs its launches in order), with every gather on
    a stream of its own; under the second placement of appends no gather stream,
    since appends that evict make each step's first launch wait for the last
    step's gathers. Any other value is returned as given."""
    if streams != "auto":
        return streams
    s = {1: "one+gather", 2: "group+gather"}.get(groups, "two+gather")
    return s.split("+")[0] if placement == "ring" else s


def code_digest(path: str) -> str:
    """sha256 of a C/C++ source with its comments removed and whitespace runs
    collapsed: it changes when the code changes, not when a comment does."""
    import hashlib
    import re
    with open(path) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return hashlib.sha256(" ".join(src.split()).encode()).hexdigest()


def gather_traffic(workload: str, mode: str = "layer"):
    """HBM bytes per gather launch from the committed rocprofv3 counter record
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy of known size), or
    None when there is no record for this workload and gather mode or the kernel
    code changed since the counters were taken."""
    suffix = "" if mode == "layer" else f"_{mode}"
    path = os.path.join(ROOT, "profiles", f"traffic_k_gather_{workload}{suffix}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "serving_pb_lru_amd", "csrc", "k_gather.hip")
    if code_digest(src) != rec["k_gather_hip_code_sha256"]:
        return None
    return rec["traffic_bytes_per_launch"]


LINK_SOURCES = ("k_select.hip", "miss_path.h", "device_util.h")


def link_code_digest() -> str:
    """Digest of the code the host-link launch (k_mark) is built from."""
    import hashlib
    parts = [code_digest(os.path.join(ROOT, "serving_pb_lru_amd", "csrc", f)) for f in LINK_SOURCES]
    return hashlib.sha256(" ".join(parts).encode()).hexdigest()


def link_traffic(workload: str):
    """Host-link bytes per k_mark launch from the committed rocprofv3 counter record
    (IO read and write requests of the L2, in 32-byte units), as {"read", "write"},
    or None when there is no record for this workload or the kernel's code changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_k_mark_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("k_mark_code_sha256") != link_code_digest():
        return None
    return rec["traffic_bytes_per_launch"]


def rows_per_step(tr) -> int:
    wl = tr.wl
    return wl.groups * tr.n_sets * tr.k * wl.layers


# ---------------------------------------------------------------------------
_T0 = time.perf_counter()


def note(msg: str) -> None:
    """A progress line on stderr (the JSON result is the only line on stdout)."""
    print(f"[bench {time.perf_counter() - _T0:7.1f}s] {msg}", file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _rows_chunk(args):
    from synth import rows_for
    seed, g, las, layers, row_bytes = args
    return rows_for(seed, g, las, layers, row_bytes)


def _loaded_group(tr, g: int, workers: int, placement: str = "lowest"):
    """The oracle's group g after the initial load, in full-data mode. The rows
    (inputs from synth) are generated by `workers` processes; the oracle appends
    them chunk by chunk in load order, as oracle.replay.initial_load does."""
    import multiprocessing as mp

    from oracle.replay import LOAD_CHUNK, new_group
    wl = tr.wl
    grp = new_group(tr, full_data=True, placement=placement)
    order = tr.initial_load_order()
    spans = [(s, min(s + LOAD_CHUNK, order.size)) for s in range(0, order.size, LOAD_CHUNK)]
    jobs = [(wl.seed, g, order[s:e], wl.layers, wl.row_bytes) for s, e in spans]
    with mp.get_context("fork").Pool(max(1, workers)) as pool:
        for (s, e), rows in zip(spans, pool.imap(_rows_chunk, jobs, chunksize=1)):
            grp.append(order[s:e], rows)
    return grp


def _oracle_step(grp, tr, g: int, t: int, sel, app_rows):
    """One decode step of group g on the oracle: appends, step, every layer's gather."""
    grp.append(tr.appends(t), app_rows)
    grp.step(sel)
    for l in range(tr.wl.layers):
        grp.gather(sel, l, step=t)


def _timed_steps(grp, tr, g: int, sels, first: int, count: int, core: int, conn) -> None:
    """Child process: pinned to `core`, time steps first .. first+count-1 of group g
    (the appended rows are generated before each step's clock starts); send
    (row-layers, seconds) back."""
    from synth import rows_for
    os.sched_setaffinity(0, {core})
    wl = tr.wl
    rows, spent = 0, 0.0
    for t in range(first, first + count):
        sel = next(sels)
        app_rows = rows_for(wl.seed, g, tr.appends(t), wl.layers, wl.row_bytes)
        t0 = time.perf_counter()
        _oracle_step(grp, tr, g, t, sel, app_rows)
        spent += time.perf_counter() - t0
        rows += tr.n_sets * tr.k * wl.layers
    conn.send((rows, spent))
    conn.close()


def _fork_timed(jobs):
    """Run _timed_steps jobs [(grp, tr, g, sels, first, count, core)] in forked
    children at once; returns [(row-layers, seconds, wall)] per job."""
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    procs = []
    t0 = time.perf_counter()
    for job in jobs:
        rd, wr = ctx.Pipe(duplex=False)
        p = ctx.Process(target=_timed_steps, args=(*job, wr))
        p.start()
        wr.close()
        procs.append((p, rd))
    out = []
    for p, rd in procs:
        rows, spent = rd.recv()
        p.join()
        if p.exitcode != 0:
            raise RuntimeError(f"oracle replay process failed ({p.exitcode})")
        out.append((rows, spent))
    wall = time.perf_counter() - t0
    return [(r, s, wall) for r, s in out]


def cpu_baseline(tr, W: int, K: int, seconds: float, parallel: bool = True,
                 placement: str = "lowest") -> dict:
    """The oracle (full-data mode: rows moved and gathered) timed on this host's cores.

    Protocol: the initial load and W warm-up steps are untimed (the load's row
    generation runs on every core; the oracle itself is single-threaded). From the
    warmed state, three replays of the same steps W+1 .. W+Kc each run in a
    forked child pinned to one core (a fork copies the state, so every replay
    starts from the same point, as a fresh start would); the median replay is the
    single-core figure. Kc is chosen so the three replays take about `seconds` of
    CPU work (at most K). Groups are independent, so a second figure runs
    min(G, cores) groups at once, one per core (each from its own warmed state),
    when their pools fit in half the free host memory: rows/s summed over
    processes, over the wall time of the slowest."""
    import statistics

    from synth import rows_for
    wl = tr.wl
    cores = sorted(os.sched_getaffinity(0))
    per_group_bytes = (tr.P + tr.H) * wl.layers * wl.row_bytes
    avail = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable"):
                    avail = int(line.split()[1]) * 1024
    except OSError:
        pass
    n_par = min(wl.groups, len(cores)) if parallel else 1
    if avail is not None:
        n_par = max(1, min(n_par, int(0.5 * avail // max(per_group_bytes * 1.3, 1))))
    t_load = time.perf_counter()
    warmed = []
    est = None
    first_s = None
    for g in range(n_par):
        grp = _loaded_group(tr, g, len(cores), placement)
        sels = tr.selections(g)
        t_w = time.perf_counter()
        for t in range(1, W + 1):
            sel = next(sels)
            app_rows = rows_for(wl.seed, g, tr.appends(t), wl.layers, wl.row_bytes)
            t_s = time.perf_counter()
            _oracle_step(grp, tr, g, t, sel, app_rows)
            if g == 0 and t == 1:
                first_s = time.perf_counter() - t_s
        if g == 0 and W:
            est = (time.perf_counter() - t_w) / W
        warmed.append((grp, sels))
        note(f"cpu baseline: group {g} loaded and warmed ({time.perf_counter() - t_load:.1f}s so far)")
    load_s = time.perf_counter() - t_load
    kc = K if not est else max(1, min(K, int(round(seconds / 3 / est))))
    grp0, sels0 = warmed[0]
    single = []
    for _ in range(3):
        rows, spent, _ = _fork_timed([(grp0, tr, 0, sels0, W + 1, kc, cores[0])])[0]
        single.append(rows / spent)
        note(f"cpu baseline: replay {len(single)}: {kc} steps in {spent:.1f}s")
    res = {"value": round(statistics.median(single), 1), "unit": "rows/s", "cores": 1, "kind": "oracle",
           "cpu_model": cpu_model(), "host_cores": len(cores),
           "replays": [round(v, 1) for v in single],
           "sample": (f"{wl.name} group 0 of {wl.groups}: steps {W + 1}..{W + kc} of the trace timed "
                      f"(load and {W} warm-up steps untimed), median of 3 replays from the same warmed "
                      f"state, each in a process pinned to one core; full-data mode (rows moved and "
                      f"gathered)")}
    if n_par > 1:
        jobs = [(grp, tr, g, sels, W + 1, kc, cores[g % len(cores)]) for g, (grp, sels) in enumerate(warmed)]
        out = _fork_timed(jobs)
        total_rows = sum(r for r, _, _ in out)
        wall = max(w for _, _, w in out)
        res["parallel"] = {"value": round(total_rows / wall, 1), "unit": "rows/s", "cores": n_par,
                           "sample": f"groups 0..{n_par - 1} at once, one process per core, steps "
                                     f"{W + 1}..{W + kc} each"}
    elif wl.groups > 1:
        res["parallel"] = {"value": None, "note": "the groups' full-data pools do not fit in half the free "
                                                  "host memory together"}
    res["untimed_setup_s"] = round(load_s, 1)
    if first_s is not None:   # the cold start, apart from the steady steps (not pinned to a core)
        res["first_step_s"] = round(first_s, 3)
    return res


# ---------------------------------------------------------------------------
def gather_all_layers(eng, g, sel, outs, layers, mode, stream=None):
    """Every layer of group g's selection into outs ([layers][n_sets][k][row_bytes]):
    one ula_gather per layer, layer 0 alone and the later layers in one
    ula_gather_layers launch ("split"), or all layers in one launch ("all")."""
    if mode == "layer":
        for l in range(layers):
            eng.gather(g, l, sel, out=outs[l], stream=stream)
    elif mode == "all":
        eng.gather_layers(g, 0, layers, sel, out=outs, stream=stream)
    else:
        eng.gather(g, 0, sel, out=outs[0], stream=stream)
        if layers > 1:
            eng.gather_layers(g, 1, layers - 1, sel, out=outs[1:], stream=stream)


def gpu_run(tr, W: int, K: int, phases: bool, policy: int = 0, gather_mode: str = "layer",
            replays: int = 3, placement: int = 0, streams: str = "one", group0: int = 0) -> dict:
    """group0: engine group g runs the workload's group group0 + g (its rows and selections)."""
    import statistics

    import torch

    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device

    wl = tr.wl
    groups = list(range(wl.groups))
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()   # a created stream: launches on the legacy null stream cost more
    torch.cuda.set_stream(stream)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, group0 + g)

    # inputs for every step, resident in HBM before timing
    sels = {g: [torch.from_numpy(s).cuda() for s in tr.selections(group0 + g)] for g in groups}
    apps = [tr.appends(t) for t in range(1, tr.steps + 1)]
    app_rows = {g: [rows(a, g) for a in apps] for g in groups}
    # one buffer per group: its layers' gathered rows one after the other
    outs = {g: torch.empty((wl.layers, tr.n_sets, tr.k, wl.row_bytes), dtype=torch.uint8, device="cuda")
            for g in groups}

    if streams.startswith("group"):
        gstreams = [torch.cuda.Stream() for _ in groups]
    elif streams.startswith("two"):
        pair = [torch.cuda.Stream(), torch.cuda.Stream()]
        gstreams = [pair[g % 2] for g in groups]
    elif streams == "one+gather":
        one = torch.cuda.Stream()
        gstreams = [one for _ in groups]
    else:
        gstreams = [stream for _ in groups]
    side = [gs for i, gs in enumerate(gstreams) if gs is not stream and gs not in gstreams[:i]]
    # X+gather: the gathers go to the main stream, after an event their step
    # recorded (the library orders the group's next swap after them)
    gather_stream = stream if streams.endswith("+gather") else None
    step_done = {g: torch.cuda.Event() for g in groups}

    def fork():   # the group streams start after what the main stream has recorded
        for gs in side:
            gs.wait_stream(stream)

    def join():   # and the main stream continues after all of them
        for gs in side:
            stream.wait_stream(gs)

    def run_step(eng, t):
        for g in groups:
            sel = sels[g][t - 1]
            # the step's appends and the step in one call (the appends run in the
            # step's first launch when they are small)
            if gather_stream is None:
                eng.append_step(g, apps[t - 1], app_rows[g][t - 1], sel, stream=gstreams[g])
                gather_all_layers(eng, g, sel, outs[g], wl.layers, gather_mode, stream=gstreams[g])
            else:
                eng.append_step(g, apps[t - 1], app_rows[g][t - 1], sel, stream=gstreams[g])
                step_done[g].record(gstreams[g])
                gather_stream.wait_event(step_done[g])
                gather_all_layers(eng, g, sel, outs[g], wl.layers, gather_mode, stream=gather_stream)

    # every step kernel runs once on a tiny engine first, so that the first
    # timed step does not also pay for loading kernel code
    tiny = Trace(dataclasses.replace(preset("tiny_4x4k"), layers=wl.layers, groups=1), steps=2)
    warm = engine_for(tiny, max_append=1 << 12, policy=policy)
    initial_load(warm, tiny, [0], lambda las, g: rows_device(las, wl.layers, tiny.wl.row_bytes, 0, g))
    for t, sel in enumerate(tiny.selections(0), start=1):
        app = tiny.appends(t)
        dsel = torch.from_numpy(sel).cuda()
        warm.append_step(0, app, rows_device(app, wl.layers, tiny.wl.row_bytes, 0, 0), dsel)
        gather_all_layers(warm, 0, dsel, torch.empty((wl.layers, tiny.n_sets, tiny.k, tiny.wl.row_bytes),
                                                     dtype=torch.uint8, device="cuda"), wl.layers, gather_mode)
    warm.sync()
    warm.close()

    def timed_replay(timed_kernels: bool):
        eng = engine_for(tr, max_append=1 << 16, policy=policy, placement=placement)
        initial_load(eng, tr, groups, rows)
        torch.cuda.synchronize()
        # the first step (cold start: the most misses) is timed on its own
        s1, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        first_ms = None
        for t in range(1, W + 1):
            if t == 1:
                s1.record()
                fork()
            run_step(eng, t)
            if t == 1:
                join()
                e1.record()
                torch.cuda.synchronize()
                first_ms = s1.elapsed_time(e1)
        torch.cuda.synchronize()
        # timed_kernels: every gather and every step's host-link launch (k_mark) of
        # the timed region records its kernel's start and end in its own dispatch
        # (HIP events on the launch's stream, no launch overhead inside; they cost
        # the host 6-13 us per launch to enqueue)
        eng.set_timing(eng.TIMING_GATHER | eng.TIMING_LINK if timed_kernels else 0)
        eng.read_gather_timing()
        eng.read_link_timing()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        fork()
        t0 = time.perf_counter()
        for t in range(W + 1, W + K + 1):
            run_step(eng, t)
        join()
        end.record()
        enqueue = time.perf_counter() - t0   # the host's time to enqueue the K steps
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        eng.sync()   # raises if the device latched an error
        g_ms, g_n = eng.read_gather_timing()
        l_ms, l_n = eng.read_link_timing()
        eng.set_timing(0)
        eng.close()
        return dict(wall_s=wall, enqueue_s=enqueue, event_ms=start.elapsed_time(end), gather_ms=g_ms / max(g_n, 1),
                    gather_launches=g_n, link_ms=l_ms / max(l_n, 1), link_launches=l_n, first_step_ms=first_ms)

    # the replays that give the value carry no timing events; one more replay of
    # the same steps, with them, gives the kernels' live durations
    runs = []
    for i in range(max(1, replays)):
        runs.append(timed_replay(False))
        note(f"gpu replay {i + 1}: {runs[-1]['event_ms'] / K:.4f} ms per step")
    order = sorted(range(len(runs)), key=lambda i: runs[i]["wall_s"])
    res = dict(runs[order[len(order) // 2]])   # the median replay
    res["replay_walls_s"] = [r["wall_s"] for r in runs]
    inst = timed_replay(True)
    note(f"gpu replay with kernel timing: {inst['event_ms'] / K:.4f} ms per step")
    for key in ("gather_ms", "gather_launches", "link_ms", "link_launches"):
        res[key] = inst[key]
    res["instrumented_ms_per_step"] = inst["event_ms"] / K

    # ---- per-phase replay (diagnostic, synchronises every step) --------------
    # also the step statistics: the host-link bytes of the timed steps (the engine
    # is deterministic, so they are those of the timed replays)
    if phases:
        eng = engine_for(tr, max_append=1 << 16, policy=policy, placement=placement)
        initial_load(eng, tr, groups, rows)
        eng.set_timing(eng.TIMING_STEP | eng.TIMING_GATHER)
        torch.cuda.synchronize()
        ph = np.zeros(3)
        h2d = d2h = hits = uniq = 0
        n = 0
        prev_evict = {g: 0 for g in groups}
        for t in range(1, W + K + 1):
            if t == W + 1:
                eng.read_gather_timing()   # from here on: the timed steps' gathers
            for g in groups:
                eng.append_step(g, apps[t - 1], app_rows[g][t - 1], sels[g][t - 1])
                # the gathers alone: one group at a time, right behind its step on
                # the same stream (as in the timed steps, so no idle queue before them)
                gather_all_layers(eng, g, sels[g][t - 1], outs[g], wl.layers, gather_mode)
                # [0] includes a small append (it runs in the lookup's first launch);
                # [1] also moves this step's misses in, last step's evictions out
                ms = eng.read_timing(g)
                st = eng.sync()[g]
                if t > W:
                    ph += ms
                    h2d += st[2]
                    d2h += prev_evict[g]
                    hits += st[1]
                    uniq += st[0]
                    n += 1
                prev_evict[g] = st[3]
        g_alone_ms, g_alone_n = eng.read_gather_timing()
        eng.close()
        note("gpu per-phase replay done")
        res.update(gather_alone_ms=g_alone_ms / max(g_alone_n, 1), gather_alone_launches=g_alone_n)
        res.update(phase_ms=(ph / max(n, 1)).tolist(), link_ms_total=float(ph[1]),
                   h2d_rows=int(h2d), d2h_rows=int(d2h), group_steps=n,
                   hit_rate=hits / uniq if uniq else None)
    return res


def copy_peaks(gib: float = 1.0) -> dict:
    """hipMemcpyAsync between pinned host memory and HBM: GB/s host-to-device,
    device-to-host, and each direction when both run at once (two streams)."""
    import torch
    n = int(gib * (1 << 30))
    h_in = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    h_out = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    d_in = torch.empty(n, dtype=torch.uint8, device="cuda")
    d_out = torch.empty(n, dtype=torch.uint8, device="cuda")
    s_a, s_b = torch.cuda.Stream(), torch.cuda.Stream()

    def run(copies):
        for _ in range(2):   # the first copies page the buffers in
            for s, fn in copies:
                with torch.cuda.stream(s):
                    fn()
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s, fn in copies:
            with torch.cuda.stream(s):
                fn()
        torch.cuda.synchronize()
        return n / (time.perf_counter() - t0) / 1e9

    h2d = run([(s_a, lambda: d_in.copy_(h_in, non_blocking=True))])
    d2h = run([(s_a, lambda: h_out.copy_(d_out, non_blocking=True))])
    both = run([(s_a, lambda: d_in.copy_(h_in, non_blocking=True)),
                (s_b, lambda: h_out.copy_(d_out, non_blocking=True))])
    return {"bytes": n, "h2d": round(h2d, 2), "d2h": round(d2h, 2), "bidirectional_each": round(both, 2)}


def layer_prefetch(tr, W: int, K: int, compute_us: float) -> list:
    """Later-layer prefetch on a second stream (UlaCache summary, section 2: one
    lookup and de-duplication serves a whole layer group, and a second stream
    brings in the group's later layers during the compute of an earlier one). Here a step moves every layer of a missed entry at once, so the
    later layers' gathers are what a second stream can take off the critical path.

    Two schedules of the same steps, each group's layers followed by a synthetic
    per-layer compute of `compute_us`:
      serial    one stream: step, then per layer gather and compute;
      prefetch  the step and layer 0's gather on the main stream; layers 1.. gathered
                on a second stream ordered after the step by an event; layer l's
                compute waits for its gather's event;
      prefetch_one_launch  as prefetch, with layers 1.. gathered by one
                ula_gather_layers launch (one event for all of them);
      prefetch_flag  as prefetch_one_launch, but the second stream is gated on the
                device by the group's completion counter (hipStreamWaitValue64 on
                ula_flag_address reaching the step) instead of an event recorded
                after the step on the main stream.
    Two stand-ins for the compute: a single-lane spin (occupies no resources: the
    upper bound of what overlap can hide) and a bf16 matrix product sized to the
    same duration (occupies the matrix cores of the whole chip, like attention
    math). Returns one result per stand-in."""
    import torch

    from serving_pb_lru_amd.replay import engine_for, initial_load
    from synth.device import rows_device

    wl = tr.wl
    groups = list(range(wl.groups))
    torch.cuda.set_device(0)
    main_s = torch.cuda.Stream()
    side_s = torch.cuda.Stream()
    torch.cuda.set_stream(main_s)
    rows = lambda las, g: rows_device(las, wl.layers, wl.row_bytes, wl.seed, g)
    sels = {g: [torch.from_numpy(s).cuda() for s in tr.selections(g)] for g in groups}
    apps = [tr.appends(t) for t in range(1, tr.steps + 1)]
    app_rows = {g: [rows(a, g) for a in apps] for g in groups}
    outs = {g: torch.empty((wl.layers, tr.n_sets, tr.k, wl.row_bytes), dtype=torch.uint8, device="cuda")
            for g in groups}

    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    # stand-ins calibrated to compute_us
    spin_us_per_kcycle = timed(lambda: torch.cuda._sleep(100000)) / 100.0
    spin_cycles = int(compute_us / spin_us_per_kcycle * 1000)
    best = None
    for n in (512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192):
        x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        y = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        us = timed(lambda: torch.mm(x, y))
        if best is None or abs(us - compute_us) < abs(best[1] - compute_us):
            best = (n, us, x, y)
    n_mm, mm_us, xa, xb = best
    stand_ins = {"spin": (lambda: torch.cuda._sleep(spin_cycles), timed(lambda: torch.cuda._sleep(spin_cycles))),
                 "bf16_matmul": (lambda: torch.mm(xa, xb), mm_us)}

    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")   # the HIP runtime torch has loaded
    hip.hipStreamWaitValue64.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint,
                                         ctypes.c_uint64]
    hip.hipStreamWaitValue64.restype = ctypes.c_int
    WAIT_GTE = 0x0

    results = []
    for kind, (compute, c_us) in stand_ins.items():
        per = {}
        for sched in ("serial", "prefetch", "prefetch_one_launch", "prefetch_flag"):
            eng = engine_for(tr, max_append=1 << 16)
            initial_load(eng, tr, groups, rows)
            torch.cuda.synchronize()
            flags = [eng.flag_address(g) for g in groups]

            def step(t):
                for g in groups:
                    sel = sels[g][t - 1]
                    eng.append_step(g, apps[t - 1], app_rows[g][t - 1], sel)
                    if sched == "serial":
                        for l in range(wl.layers):
                            eng.gather(g, l, sel, out=outs[g][l])
                            compute()
                        continue
                    eng.gather(g, 0, sel, out=outs[g][0])
                    if sched == "prefetch_flag":
                        # the step of group g is its t-th: wait on the device for its
                        # counter (a failed step sets a bit that also releases this)
                        rc = hip.hipStreamWaitValue64(ctypes.c_void_p(side_s.cuda_stream),
                                                      ctypes.c_void_p(flags[g]), t, WAIT_GTE,
                                                      0xFFFFFFFFFFFFFFFF)
                        assert rc == 0, rc
                    else:
                        after_step = torch.cuda.Event()
                        after_step.record(main_s)
                        side_s.wait_event(after_step)
                    ready = []
                    if sched in ("prefetch_one_launch", "prefetch_flag") and wl.layers > 1:
                        eng.gather_layers(g, 1, wl.layers - 1, sel, out=outs[g][1:], stream=side_s)
                        ev = torch.cuda.Event()
                        ev.record(side_s)
                        ready = [ev] + [None] * (wl.layers - 2)
                    else:
                        for l in range(1, wl.layers):
                            eng.gather(g, l, sel, out=outs[g][l], stream=side_s)
                            ev = torch.cuda.Event()
                            ev.record(side_s)
                            ready.append(ev)
                    compute()
                    for ev in ready:
                        if ev is not None:
                            main_s.wait_event(ev)
                        compute()

            for t in range(1, W + 1):
                step(t)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            t0 = time.perf_counter()
            for t in range(W + 1, W + K + 1):
                step(t)
            host = (time.perf_counter() - t0) / K
            b.record()
            torch.cuda.synchronize()
            eng.sync()
            per[sched] = a.elapsed_time(b) / K
            per[sched + "_host"] = host * 1e3
            eng.close()
        results.append({
            "experiment": "later-layer prefetch on a second stream", "workload": wl.name,
            "compute": kind, "compute_us_per_layer": round(c_us, 2),
            "matmul_n": n_mm if kind == "bf16_matmul" else None,
            "layers_per_group": wl.layers, "groups": wl.groups, "steps": K, "warmup": W,
            "serial_ms_per_step": round(per["serial"], 5), "prefetch_ms_per_step": round(per["prefetch"], 5),
            "prefetch_one_launch_ms_per_step": round(per["prefetch_one_launch"], 5),
            "prefetch_flag_ms_per_step": round(per["prefetch_flag"], 5),
            "hidden_us_per_step_flag": round((per["serial"] - per["prefetch_flag"]) * 1e3, 2),
            "hidden_us_per_step": round((per["serial"] - per["prefetch"]) * 1e3, 2),
            "hidden_us_per_step_one_launch": round((per["serial"] - per["prefetch_one_launch"]) * 1e3, 2),
            "host_enqueue_ms_per_step": {k: round(per[k + "_host"], 5)
                                         for k in ("serial", "prefetch", "prefetch_one_launch",
                                                   "prefetch_flag")},
            "compute_only_ms_per_step": round(c_us * wl.layers * wl.groups * 1e-3, 5)})
    return results


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.copy_ceiling:
        copy_ceiling(args.copy_ceiling)
        return
    if args.copy_probe:
        from measure import probes
        rows = [int(x) for x in args.copy_probe.split(",")]
        print(json.dumps({"probe": "copy", **probes.copy(rows, args.slot_bytes)}), flush=True)
        return
    if args.link_probe or args.gather_probe:
        from measure import probes
        if args.link_probe:
            r = probes.link(args.link_probe, args.slot_bytes, args.pool_rows or 8 * args.link_probe)
        else:
            r = probes.gather(args.gather_probe, args.slot_bytes, args.pool_rows or 4 * args.gather_probe)
        print(json.dumps({"probe": "link" if args.link_probe else "gather", **r}), flush=True)
        return
    if args.layer_prefetch:
        wl = preset(args.workload)
        tr = Trace(wl, steps=max(args.warmup + args.steps, 1))
        for r in layer_prefetch(tr, args.warmup, args.steps, args.layer_prefetch):
            print(json.dumps(r), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the engine is the single-GPU DP form; each GPU of a node would run its own "
              "independent engine over its own requests.", file=sys.stderr)
        sys.exit(2)
    W, K = args.warmup, args.steps
    wl = preset(args.workload)
    groups_total = wl.groups
    if args.groups:
        # the first N groups are the same traces as in the full workload (each
        # group's selections come from its own seeded stream)
        wl = dataclasses.replace(wl, groups=min(args.groups, wl.groups))
    g0 = args.first_group
    if g0:
        if not args.groups or not 0 < g0 < groups_total:
            print(f"--first-group {g0} needs --groups and 0 < G0 < {groups_total}", file=sys.stderr)
            sys.exit(2)
        wl = dataclasses.replace(wl, groups=min(args.groups, groups_total - g0))
    tr = Trace(wl, steps=max(W + K, 1))
    per_step = rows_per_step(tr)

    policy = 1 if args.policy == "lru" else 0
    cpu = None
    if not args.no_cpu_baseline and policy == 0 and not g0:
        cpu = cpu_baseline(tr, W, K, args.cpu_seconds, parallel=not args.no_cpu_parallel,
                           placement=args.placement)

    gather_mode = args.gather if wl.layers > 1 else "layer"   # one layer: the same launch
    streams = schedule_for(wl.groups, args.placement, args.streams)
    placement = 1 if args.placement == "ring" else 0
    r = gpu_run(tr, W, K, not args.no_phases, policy, gather_mode, replays=args.replays,
                placement=placement, streams=streams, group0=g0)
    value = per_step * K / r["wall_s"]
    ms_per_step = r["event_ms"] / K
    replay_values = [round(per_step * K / w, 1) for w in r["replay_walls_s"]]
    rnd = lambda x, d: None if x is None else round(x, d)

    # ---- the gather against HBM peak ------------------------------------------
    # its own duration: from the per-phase replay, where every gather runs alone
    # (in the timed steps a group's gathers run beside another group's host-link
    # launch, hidden under it and slowed by it)
    g_ms = float(r.get("gather_alone_ms") or r["gather_ms"])
    # algorithmic bytes per launch: every gathered row-layer of the timed region
    # over the gather launches that moved them
    launches_per_group_step = {"layer": wl.layers, "all": 1, "split": 2}[gather_mode]
    g_bytes = 2 * wl.row_bytes * tr.n_sets * tr.k * wl.layers / launches_per_group_step
    assert r["gather_launches"] == K * wl.groups * launches_per_group_step, r["gather_launches"]
    if "gather_alone_launches" in r:
        assert r["gather_alone_launches"] == K * wl.groups * launches_per_group_step, r["gather_alone_launches"]
    g_gbs = g_bytes / (g_ms * 1e-3) / 1e9
    gather_line = {"bound": "hbm", "kernel": "k_gather", "achieved": round(g_gbs, 1), "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": round(g_gbs / HBM_PEAK_GBS, 4),
                   "traffic": None if g0 else gather_traffic(wl.name, gather_mode),
                   "bytes_per_launch": round(g_bytes), "launch_ms": round(g_ms, 5),
                   "launch_ms_in_timed_steps": round(float(r["gather_ms"]), 5),
                   "measured": "alone (per-phase replay)" if r.get("gather_alone_ms") else "timed steps",
                   "layers_per_launch": round(wl.layers / launches_per_group_step, 3)}

    # ---- the host-link launch (k_mark) against the link's per-direction peak ---
    link_line = None
    miss = None
    if "phase_ms" in r:
        slot = wl.layers * wl.row_bytes
        up = r["h2d_rows"] * slot          # missed rows in, over the timed steps
        down = r["d2h_rows"] * slot        # the previous steps' evicted rows out
        launches = r["link_launches"]
        assert launches == K * wl.groups, launches
        l_ms = float(r["link_ms"])
        per_launch = max(up, down) / launches
        l_gbs = per_launch / (l_ms * 1e-3) / 1e9 if l_ms > 0 else None
        link_line = {"bound": "host-link", "kernel": "k_lru_pass (first pass)" if policy else "k_mark",
                     "achieved": rnd(l_gbs, 2), "peak": round(LINK_PEAK_GBS, 1), "unit": "GB/s per direction",
                     "frac": rnd(None if l_gbs is None else l_gbs / LINK_PEAK_GBS, 4),
                     "traffic": None,
                     "bytes_per_launch": round(per_launch),
                     "h2d_bytes_per_launch": round(up / launches), "d2h_bytes_per_launch": round(down / launches),
                     "launch_ms": round(l_ms, 5),
                     "note": "max-direction algorithmic bytes (656 x layers per missed row in, per "
                             "evicted row of the previous step out; both directions move "
                             "concurrently) over the launch's average duration, which also marks "
                             "hits and plans and extracts the victims"}
        counted = link_traffic(wl.name) if not policy and not g0 else None
        if counted:   # counted host-link bytes per launch, the roofline's direction and both
            link_line["traffic"] = counted["read"] if up >= down else counted["write"]
            link_line["traffic_read_write"] = [counted["read"], counted["write"]]
        t_in = r["link_ms_total"] * 1e-3
        gin = up / t_in / 1e9 if t_in > 0 else None
        gout = down / t_in / 1e9 if t_in > 0 else None
        miss = {"hit_rate": rnd(r["hit_rate"], 6),
                "phase_ms_per_group_step": {k: round(v, 5) for k, v in zip(
                    ["lookup_dedup", "mark_select_link", "swap_commit"], r["phase_ms"])},
                "h2d_GBps_over_phase": rnd(gin, 2), "d2h_GBps_over_phase": rnd(gout, 2)}
        try:
            peaks = copy_peaks()
            miss["measured_copy_peak_GBps"] = peaks
            if l_gbs is not None and peaks["bidirectional_each"]:
                miss["link_frac_of_measured_bidirectional_copy"] = round(l_gbs / peaks["bidirectional_each"], 4)
        except RuntimeError as e:   # pinned memory refused: report without the measured peaks
            miss["measured_copy_peak_GBps"] = f"not measured: {e}"
    # the dominant kernel of the step: the host-link launch when the step moves
    # rows over the link for longer than it gathers, else the gather
    link_dominant = link_line is not None and link_line["launch_ms"] > gather_line["launch_ms"] * \
        launches_per_group_step
    roofline, other = (link_line, gather_line) if link_dominant else (gather_line, link_line)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "rows/s", "n_gpus": 1, "steps": K,
        "selections_per_s": round(value / wl.layers, 1),
        "first_step_ms": None if r.get("first_step_ms") is None else round(r["first_step_ms"], 5),
        "warmup": W, "ms_per_step": round(ms_per_step, 5),
        "host_enqueue_ms_per_step": round(r["enqueue_s"] * 1e3 / K, 5),
        "instrumented_ms_per_step": round(r["instrumented_ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": wl.name, "requests": wl.requests,
                   "context": wl.ctx_fixed if wl.ctx_fixed else list(wl.ctx_range),
                   "sets_per_request": wl.sets_per_request, "groups": wl.groups,
                   "groups_of_workload": groups_total, **({"first_group": g0} if g0 else {}),
                   "layers_per_group": wl.layers, "k": wl.k, "gpu_slots": tr.P, "host_slots": tr.H,
                   "ring": wl.ring, "row_bytes": wl.row_bytes, "overlap": wl.overlap,
                   "policy": "exact LRU" if policy else "PB-LRU", "gather": gather_mode,
                   "placement": args.placement, "streams": streams,
                   "row_layers_per_step": per_step},
        "roofline": roofline,
        "roofline_other": other,
        "replays": replay_values,
        "miss_path": miss,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
