// Host runtime of the residency engine: configuration checks, workspace
// layout, launch sequencing on the caller's stream, error latching and state
// export. Implements the C ABI declared in include/ula.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ula_internal.h"

using namespace ula;

namespace {

constexpr size_t kAlign = 256;
constexpr int kStageSlots = 4;   // pinned staging buffers per group for appended addresses

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

thread_local std::string g_hip_error;

int hip_fail(hipError_t e, const char* what) {
  g_hip_error = std::string(what) + ": " + hipGetErrorString(e);
  return ULA_EHIP;
}

#define HIP_TRY(expr)                                 \
  do {                                                \
    hipError_t e_ = (expr);                           \
    if (e_ != hipSuccess) return hip_fail(e_, #expr); \
  } while (0)

struct Dims {
  int64_t N, P, H, B, NB, W, T, WH, TH, Lg, row_bytes, slot_bytes;
  int64_t maxU, maxBlk, maxItems, maxApp, nsel, maxRs;
  int policy, placement;
};

bool check_config(const ula_config* c, Dims* d) {
  if (!c) return false;
  if (c->num_groups < 1 || c->num_groups > 4096) return false;
  if (c->layers_per_group < 1 || c->layers_per_group > 256) return false;
  if (c->row_bytes < 16 || c->row_bytes > 4096 || c->row_bytes % 16) return false;
  if (c->ring_buckets < 1 || c->ring_buckets > kMaxRing) return false;
  if (c->logical_capacity < 1) return false;
  if (c->gpu_slots < 1 || c->host_slots < 0) return false;
  if ((int64_t)c->gpu_slots + c->host_slots >= (1ll << 31)) return false;
  if (c->max_sets < 1 || c->max_k < 1 || c->max_append < 1) return false;
  if (c->policy != ULA_POLICY_PBLRU && c->policy != ULA_POLICY_LRU) return false;
  if (c->placement != ULA_PLACE_LOWEST && c->placement != ULA_PLACE_RING) return false;
  if (c->placement == ULA_PLACE_RING && c->policy != ULA_POLICY_PBLRU) return false;
  const int64_t nsel = (int64_t)c->max_sets * c->max_k;
  if (nsel >= (1ll << 31)) return false;
  d->N = c->logical_capacity;
  d->P = c->gpu_slots;
  d->H = c->host_slots;
  d->B = c->ring_buckets;
  d->NB = d->B + 2;
  d->W = (d->P + 31) / 32;
  d->T = (d->W + kTileWords - 1) / kTileWords;
  d->WH = (d->H + 31) / 32;
  d->TH = (d->WH + kTileWords - 1) / kTileWords;
  d->Lg = c->layers_per_group;
  d->row_bytes = c->row_bytes;
  d->slot_bytes = d->Lg * d->row_bytes;
  d->maxU = std::min<int64_t>(nsel, d->P);
  d->nsel = nsel;
  d->maxBlk = (nsel + kScanBlock - 1) / kScanBlock;
  d->maxApp = c->max_append;
  // an append under placement ring takes up to two outputs per entry (its GPU
  // slot and a host slot for the entry it displaces), each work item at least one
  d->maxItems = std::max<int64_t>(d->maxU, 2 * d->maxApp) + 2;
  d->maxRs = (d->maxU + 1023) / 1024;
  d->policy = c->policy;
  d->placement = c->placement;
  // selection entries (and so misses) fit the look-back descriptors' 30-bit counts
  if (nsel >= (1ll << 30)) return false;
  // 16-byte piece counts handled with 32-bit indices and FastDiv (< 2^31)
  if (nsel * (d->row_bytes / 16) >= (1ll << 31)) return false;
  if (d->maxU * (d->slot_bytes / 16) >= (1ll << 31)) return false;
  if (d->maxApp * (d->slot_bytes / 16) >= (1ll << 31)) return false;
  return true;
}

struct Layout {
  size_t map, tag, gown, stamp, dirty, hown, bm, tcnt, hbm, htcnt, hits, mla, mh, vict, blk,
      partial, items, app_la, app_dst, app_rows, evict_rows, wb_h, miss_e, miss_stage, miss_rows,
      hs_stage, res, lru_ts, lru_hist, span_a, span_b, sort_key[2], sort_slot[2], rs_hist, rs_base, pool,
      group_bytes;
  size_t counters_bytes, total;
};

Layout layout_of(const ula_config* c, const Dims& d) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.map = take(4 * d.N);
  L.tag = take(8 * d.N);
  L.gown = take(4 * d.P);
  L.stamp = take(4 * 32 * d.W);
  L.dirty = take(4 * d.T);
  L.hown = take(4 * d.H);
  L.bm = take(4 * d.NB * d.W);
  L.tcnt = take(4 * d.NB * d.T);
  L.hbm = take(4 * d.WH);
  L.htcnt = take(4 * d.TH);
  L.hits = take(4 * d.maxU);
  L.mla = take(4 * d.maxU);
  L.mh = take(4 * d.maxU);
  L.vict = take(4 * d.maxU);
  L.blk = take(8 * 2 * d.maxBlk);
  L.partial = take(4 * kMarkBlocks * kMaxBuckets);
  L.items = take(sizeof(SelItem) * d.maxItems);
  L.app_la = take(4 * d.maxApp);
  L.app_dst = take(4 * 2 * d.maxApp);
  L.app_rows = take((size_t)d.maxApp * d.slot_bytes);
  L.evict_rows = take((size_t)d.maxU * d.slot_bytes);
  L.wb_h = take(4 * d.maxU);
  L.miss_e = take(4 * d.maxU);
  L.miss_stage = take(4 * d.maxU);
  L.miss_rows = take((size_t)d.maxU * d.slot_bytes);
  L.hs_stage = take(8 * d.H);
  L.res = take(8 * 2 * d.nsel);   // two buffers, by step parity
  if (d.policy == ULA_POLICY_LRU) {   // exact-LRU timestamps and selection scratch
    L.lru_ts = take(4 * 32 * d.W);
    L.lru_hist = take(4 * 2048);
    L.span_a = take(4 * d.T);
    L.span_b = take(4 * d.T);
    for (int i = 0; i < 2; ++i) {
      L.sort_key[i] = take(4 * d.maxU);
      L.sort_slot[i] = take(4 * d.maxU);
    }
    L.rs_hist = take(4 * 256 * d.maxRs);
    L.rs_base = take(4 * 256);
  }
  L.pool = take((size_t)d.P * d.slot_bytes);
  L.group_bytes = o;
  L.counters_bytes = align_up(sizeof(Counters) * c->num_groups);
  L.total = L.counters_bytes + L.group_bytes * c->num_groups;
  return L;
}

const char* kMessages[] = {
    "ok",
    "invalid argument or configuration",
    "logical address out of range or never appended",
    "logical address already appended or repeated in one append",
    "no free GPU or host slot left for the append",
    "a step selects more distinct entries than the GPU pool holds",
    "gathered entry not resident on the GPU, or its step has not completed",
    "context poisoned by an earlier device error",
    "HIP runtime error",
    "the static device workspace of this device is held by a live context",
    "the configuration needs more device workspace than the static workspace holds (32 MiB)",
};

}  // namespace

constexpr int kGatherStreams = 8;   // streams with gathers tracked per group

struct PendingGather {
  hipStream_t s = nullptr;
  hipEvent_t ev = nullptr;
  bool live = false;
};

struct GroupHost {
  GroupDev d;
  std::vector<uint64_t> appended;   // host mirror: which addresses were appended
  int64_t n_appended = 0;
  int64_t steps = 0;                // steps enqueued
  int32_t last_n = 0;               // selection entries of the last step (resolved in res)
  int32_t* stage[kStageSlots] = {};
  hipEvent_t stage_ev[kStageSlots] = {};
  bool stage_used[kStageSlots] = {};
  int stage_next = 0;
  hipEvent_t ev[4] = {};
  int32_t last_pairs = 0;           // most miss pairs the last step could have staged
  int64_t written_back = 0;         // last step whose staged rows a flush wrote to the host
  // The resolved selection (res) has two buffers, by step parity: a step writes
  // its own, the gathers of the step before read the other, so the next step's
  // lookup may run while those gathers still do.
  uint2* res_base = nullptr;
  // Gathers enqueued since the group's last row move, one event per stream: the
  // next launch that moves rows in or out of GPU slots (the swap, an append that
  // evicts, a release) waits for those on other streams.
  PendingGather pending[kGatherStreams];
};

static constexpr int kTimingRing = 256;

struct TimingRing {
  std::vector<hipEvent_t> ev;        // 2 * kTimingRing events
  int head = 0, pending = 0;
  double ms = 0.0;
  int64_t launches = 0;
};

struct ula_ctx {
  ula_config cfg;
  Dims dims;
  Layout lay;
  uint8_t* dev = nullptr;
  uint8_t* host = nullptr;
  Counters* ctrs = nullptr;
  std::vector<GroupHost> groups;
  int poisoned = 0;
  int static_dev = -1;               // device whose static workspace the context holds, or -1
  // Host-link launches of different groups share one link: once steps arrive on
  // more than one stream, each step's host-link launch records link_ev and the
  // next one on another stream waits for it, so they never run at once (the
  // rest of a group's step still overlaps another group's).
  hipStream_t first_step_stream = nullptr;
  bool multi_stream = false;
  hipEvent_t link_ev = nullptr;
  hipStream_t link_ev_stream = nullptr;   // stream of the launch link_ev last recorded
  int timing = 0;                    // ULA_TIMING_* flags
  // kernel durations of the gathers and of the steps' host-link launches: rings
  // of dispatch-recorded event pairs, summed lazily (when a ring wraps, and by
  // ula_read_gather_timing / ula_read_link_timing)
  TimingRing gather_t, link_t;
};


// ---- the static device workspace (ula_init_static) --------------------------
// For callers that cannot allocate device memory, one workspace per device lives
// in this file-scope array; each device holds its own copy for the life of the
// process. Host code never passes the array's name to a kernel or a copy (on the
// host it is only a stand-in for the symbol): it resolves the device address once
// per device with hipGetSymbolAddress, with that device current, and uses that.
constexpr size_t kStaticWorkspaceBytes = 32ull << 20;
constexpr int kMaxStaticDevices = 64;
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

static std::mutex g_static_mu;
static void* g_static_ptr[kMaxStaticDevices];     // resolved device address, per device
static bool g_static_live[kMaxStaticDevices];     // a live context holds that device's copy

// The current device's static workspace, resolved on first use, with its
// device index; claims it for one context (released by destroy_ctx).
static int claim_static_workspace(void** ptr, int* dev) {
  int d = -1;
  HIP_TRY(hipGetDevice(&d));
  if (d < 0 || d >= kMaxStaticDevices) return ULA_EINVAL;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static_live[d]) return ULA_EBUSY;
  if (!g_static_ptr[d]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (uintptr_t)p % kAlign) return ULA_EINVAL;
    g_static_ptr[d] = p;
  }
  g_static_live[d] = true;
  *ptr = g_static_ptr[d];
  *dev = d;
  return ULA_OK;
}

static void release_static_workspace(int dev) {
  if (dev < 0) return;
  std::lock_guard<std::mutex> lock(g_static_mu);
  g_static_live[dev] = false;
}

// Add the oldest pending launch's kernel time to the ring's total.
static int retire_timing(TimingRing& r) {
  const int i = (r.head - r.pending + kTimingRing) % kTimingRing;
  HIP_TRY(hipEventSynchronize(r.ev[2 * i + 1]));
  float ms = 0.f;
  HIP_TRY(hipEventElapsedTime(&ms, r.ev[2 * i], r.ev[2 * i + 1]));
  r.ms += ms;
  r.launches += 1;
  r.pending -= 1;
  return ULA_OK;
}

// The next (start, stop) event pair of a ring, for a launch that records them in
// its own dispatch (events are created on first use).
static int next_timing_pair(TimingRing& r, hipEvent_t* start, hipEvent_t* stop) {
  if (r.ev.empty()) {
    r.ev.assign(2 * kTimingRing, nullptr);
    for (auto& e : r.ev) HIP_TRY(hipEventCreate(&e));
  }
  if (r.pending == kTimingRing) {
    int rc = retire_timing(r);
    if (rc) return rc;
  }
  *start = r.ev[2 * r.head];
  *stop = r.ev[2 * r.head + 1];
  r.head = (r.head + 1) % kTimingRing;
  r.pending += 1;
  return ULA_OK;
}

// Every pending launch's time into the total; then hand the total out and reset.
static int drain_timing(TimingRing& r, double* ms, int64_t* launches) {
  while (r.pending > 0) {
    int rc = retire_timing(r);
    if (rc) return rc;
  }
  *ms = r.ms;
  *launches = r.launches;
  r.ms = 0.0;
  r.launches = 0;
  return ULA_OK;
}

// The group's resolved-selection buffer for step t (or for the gathers of step t).
static uint2* res_for(const ula_ctx* ctx, const GroupHost& gh, int64_t t) {
  return gh.res_base + (size_t)(t & 1) * (size_t)ctx->dims.nsel;
}

// A gather of the group was enqueued on stream s: record that stream's event.
// With more streams than slots, the host waits for the oldest slot's gathers.
static int note_gather(GroupHost& gh, hipStream_t s) {
  PendingGather* slot = nullptr;
  for (auto& p : gh.pending)
    if (p.live && p.s == s) slot = &p;
  for (int i = 0; !slot && i < kGatherStreams; ++i)
    if (!gh.pending[i].live) slot = &gh.pending[i];
  if (!slot) {
    slot = &gh.pending[0];
    HIP_TRY(hipEventSynchronize(slot->ev));
  }
  if (!slot->ev) HIP_TRY(hipEventCreateWithFlags(&slot->ev, hipEventDisableTiming));
  HIP_TRY(hipEventRecord(slot->ev, s));
  slot->s = s;
  slot->live = true;
  return ULA_OK;
}

// Before the first launch on stream s that moves rows in or out of the group's
// GPU slots: wait for the gathers enqueued on other streams since the last such
// launch (those on s are ordered by the stream itself).
static int wait_gathers(GroupHost& gh, hipStream_t s) {
  for (auto& p : gh.pending) {
    if (!p.live) continue;
    if (p.s != s) HIP_TRY(hipStreamWaitEvent(s, p.ev, 0));
    p.live = false;
  }
  return ULA_OK;
}

extern "C" {

size_t ula_device_bytes(const ula_config* cfg) {
  Dims d;
  if (!check_config(cfg, &d)) return 0;
  return layout_of(cfg, d).total;
}

size_t ula_host_bytes(const ula_config* cfg) {
  Dims d;
  if (!check_config(cfg, &d)) return 0;
  return (size_t)cfg->num_groups * d.H * d.slot_bytes;
}

const char* ula_strerror(int code) {
  if (code == ULA_EHIP && !g_hip_error.empty()) return g_hip_error.c_str();
  if (code > 0 || code < ULA_ETOOBIG) return "unknown error code";
  return kMessages[-code];
}

void* ula_host_alloc(size_t bytes) {
  void* p = nullptr;
  if (hipHostMalloc(&p, bytes ? bytes : 1, hipHostMallocMapped) != hipSuccess) return nullptr;
  return p;
}

int ula_host_free(void* p) {
  if (!p) return ULA_OK;
  HIP_TRY(hipHostFree(p));
  return ULA_OK;
}

static void destroy_ctx(ula_ctx* ctx) {
  release_static_workspace(ctx->static_dev);
  if (ctx->link_ev) (void)hipEventDestroy(ctx->link_ev);
  for (TimingRing* r : {&ctx->gather_t, &ctx->link_t})
    for (hipEvent_t e : r->ev)
      if (e) (void)hipEventDestroy(e);
  for (auto& g : ctx->groups) {
    for (int i = 0; i < kStageSlots; ++i) {
      if (g.stage_ev[i]) (void)hipEventDestroy(g.stage_ev[i]);
      if (g.stage[i]) (void)hipHostFree(g.stage[i]);
    }
    for (auto& e : g.ev)
      if (e) (void)hipEventDestroy(e);
    for (auto& p : g.pending)
      if (p.ev) (void)hipEventDestroy(p.ev);
  }
  delete ctx;
}

// ula_init's body. static_dev >= 0: dev_ws is that device's static workspace,
// claimed by the caller; the context then allocates no pinned staging buffers
// and no events (appends and releases copy addresses from the caller's memory,
// and step timing creates its events when it is switched on).
static int init_impl(const ula_config* cfg, void* dev_ws, void* host_pinned, uint64_t stream,
                     ula_ctx** out, int static_dev) {
  Dims d;
  if (!check_config(cfg, &d)) return ULA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  ula_ctx* ctx = new (std::nothrow) ula_ctx();
  if (!ctx) {
    release_static_workspace(static_dev);
    return ULA_EINVAL;
  }
  ctx->static_dev = static_dev;
  ctx->cfg = *cfg;
  ctx->dims = d;
  ctx->lay = layout_of(cfg, d);
  ctx->dev = static_cast<uint8_t*>(dev_ws);
  ctx->ctrs = reinterpret_cast<Counters*>(ctx->dev);
  uint8_t* hdev = nullptr;
  if (host_pinned) {
    void* p = nullptr;
    hipError_t e = hipHostGetDevicePointer(&p, host_pinned, 0);
    if (e != hipSuccess) {
      destroy_ctx(ctx);
      return hip_fail(e, "hipHostGetDevicePointer(host pool)");
    }
    hdev = static_cast<uint8_t*>(p);
  }
  ctx->host = hdev;
  ctx->groups.resize(cfg->num_groups);
  const Layout& L = ctx->lay;
  int rc = ULA_OK;
  for (int gi = 0; gi < cfg->num_groups && rc == ULA_OK; ++gi) {
    GroupHost& gh = ctx->groups[gi];
    uint8_t* b = ctx->dev + L.counters_bytes + (size_t)gi * L.group_bytes;
    GroupDev& g = gh.d;
    g.ctr = ctx->ctrs + gi;
    g.map = reinterpret_cast<uint32_t*>(b + L.map);
    g.tag = reinterpret_cast<unsigned long long*>(b + L.tag);
    g.gown = reinterpret_cast<int32_t*>(b + L.gown);
    g.stamp = reinterpret_cast<int32_t*>(b + L.stamp);
    g.dirty = reinterpret_cast<int32_t*>(b + L.dirty);
    g.hown = reinterpret_cast<int32_t*>(b + L.hown);
    g.bm = reinterpret_cast<uint32_t*>(b + L.bm);
    g.tcnt = reinterpret_cast<uint32_t*>(b + L.tcnt);
    g.hbm = reinterpret_cast<uint32_t*>(b + L.hbm);
    g.htcnt = reinterpret_cast<uint32_t*>(b + L.htcnt);
    g.hit_slots = reinterpret_cast<uint32_t*>(b + L.hits);
    g.miss_la = reinterpret_cast<int32_t*>(b + L.mla);
    g.miss_h = reinterpret_cast<uint32_t*>(b + L.mh);
    g.victims = reinterpret_cast<uint32_t*>(b + L.vict);
    g.desc = reinterpret_cast<unsigned long long*>(b + L.blk);
    g.partial = reinterpret_cast<int32_t*>(b + L.partial);
    g.items = reinterpret_cast<SelItem*>(b + L.items);
    g.app_la = reinterpret_cast<int32_t*>(b + L.app_la);
    g.app_dst = reinterpret_cast<uint32_t*>(b + L.app_dst);
    g.app_rows = b + L.app_rows;
    g.evict_rows = b + L.evict_rows;
    g.wb_h = reinterpret_cast<uint32_t*>(b + L.wb_h);
    g.miss_e = reinterpret_cast<int32_t*>(b + L.miss_e);
    g.miss_stage = reinterpret_cast<uint32_t*>(b + L.miss_stage);
    g.miss_rows = b + L.miss_rows;
    g.hs_stage = reinterpret_cast<unsigned long long*>(b + L.hs_stage);
    g.res = reinterpret_cast<uint2*>(b + L.res);
    gh.res_base = g.res;
    if (d.policy == ULA_POLICY_LRU) {
      g.lru_ts = reinterpret_cast<int32_t*>(b + L.lru_ts);
      g.lru_hist = reinterpret_cast<uint32_t*>(b + L.lru_hist);
      g.span_a = reinterpret_cast<uint32_t*>(b + L.span_a);
      g.span_b = reinterpret_cast<uint32_t*>(b + L.span_b);
      for (int i = 0; i < 2; ++i) {
        g.sort_key[i] = reinterpret_cast<uint32_t*>(b + L.sort_key[i]);
        g.sort_slot[i] = reinterpret_cast<uint32_t*>(b + L.sort_slot[i]);
      }
      g.rs_hist = reinterpret_cast<uint32_t*>(b + L.rs_hist);
      g.rs_base = reinterpret_cast<uint32_t*>(b + L.rs_base);
    }
    g.policy = d.policy;
    g.maxRs = (int32_t)std::max<int64_t>(d.maxRs, 1);
    g.pool = b + L.pool;
    g.host = hdev ? hdev + (size_t)gi * d.H * d.slot_bytes : nullptr;
    g.N = (int32_t)d.N;
    g.P = (int32_t)d.P;
    g.H = (int32_t)d.H;
    g.B = (int32_t)d.B;
    g.NB = (int32_t)d.NB;
    g.W = (int32_t)d.W;
    g.T = (int32_t)d.T;
    g.WH = (int32_t)d.WH;
    g.TH = (int32_t)d.TH;
    g.Lg = (int32_t)d.Lg;
    g.row_bytes = (int32_t)d.row_bytes;
    g.slot_bytes = (int32_t)d.slot_bytes;
    g.maxU = (int32_t)d.maxU;
    g.maxBlk = (int32_t)std::max<int64_t>(d.maxBlk, 1);
    gh.appended.assign((d.N + 63) / 64, 0);

    hipError_t e = hipSuccess;
    if (e == hipSuccess) e = launch_init_counters(g.ctr, g.P, g.H, s);
    if (e == hipSuccess) e = launch_fill_u32(g.map, d.N, kAbsent, s);
    if (e == hipSuccess) e = launch_fill_u64(g.tag, d.N, 0ull, s);
    if (e == hipSuccess) e = launch_fill_u32(reinterpret_cast<uint32_t*>(g.gown), d.P, 0xFFFFFFFFu, s);
    if (e == hipSuccess) e = launch_fill_u32(reinterpret_cast<uint32_t*>(g.stamp), 32 * d.W, 0u, s);
    if (e == hipSuccess) e = launch_fill_u32(reinterpret_cast<uint32_t*>(g.dirty), d.T, 0u, s);
    if (e == hipSuccess) e = launch_fill_u64(g.desc, 2 * g.maxBlk, 0ull, s);
    if (e == hipSuccess) e = launch_fill_u32(reinterpret_cast<uint32_t*>(g.hown), d.H, 0xFFFFFFFFu, s);
    // no host slot has a staged row: step 0xFFFFFFFF is never the previous step
    if (e == hipSuccess) e = launch_fill_u64(g.hs_stage, d.H, ~0ull, s);
    if (e == hipSuccess && g.lru_hist) e = launch_fill_u32(g.lru_hist, 2048, 0u, s);
    if (e == hipSuccess && g.lru_ts)
      e = launch_fill_u32(reinterpret_cast<uint32_t*>(g.lru_ts), 32 * d.W, 0u, s);
    if (e == hipSuccess) e = launch_fill_u32(g.bm, d.NB * d.W, 0u, s);
    if (e == hipSuccess) e = launch_fill_u32(g.tcnt, d.NB * d.T, 0u, s);
    if (e == hipSuccess) e = launch_init_bitmap(g.bm + kFree * d.W, g.W, d.P, g.tcnt + kFree * d.T, g.T, s);
    if (e == hipSuccess) e = launch_init_bitmap(g.hbm, g.WH, d.H, g.htcnt, g.TH, s);
    for (int i = 0; i < kStageSlots && e == hipSuccess && static_dev < 0; ++i) {
      e = hipHostMalloc(reinterpret_cast<void**>(&gh.stage[i]), sizeof(int32_t) * d.maxApp,
                        hipHostMallocDefault);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&gh.stage_ev[i], hipEventDisableTiming);
    }
    for (int i = 0; i < 4 && e == hipSuccess && static_dev < 0; ++i) e = hipEventCreate(&gh.ev[i]);
    if (e != hipSuccess) rc = hip_fail(e, "ula_init");
  }
  if (rc == ULA_OK) {
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) rc = hip_fail(e, "hipStreamSynchronize(init)");
  }
  if (rc != ULA_OK) {
    destroy_ctx(ctx);
    return rc;
  }
  *out = ctx;
  return ULA_OK;
}

int ula_init(const ula_config* cfg, void* dev_ws, void* host_pinned, uint64_t stream,
             ula_ctx** out) {
  if (!out) return ULA_EINVAL;
  *out = nullptr;
  Dims d;
  if (!check_config(cfg, &d)) return ULA_EINVAL;
  if (!dev_ws || ((uintptr_t)dev_ws % kAlign)) return ULA_EINVAL;
  if (d.H > 0 && !host_pinned) return ULA_EINVAL;
  return init_impl(cfg, dev_ws, host_pinned, stream, out, -1);
}

int ula_init_static(const ula_config* cfg, void* host_pinned, uint64_t stream, ula_ctx** out) {
  if (!out) return ULA_EINVAL;
  *out = nullptr;
  Dims d;
  if (!check_config(cfg, &d)) return ULA_EINVAL;
  if (layout_of(cfg, d).total > kStaticWorkspaceBytes) return ULA_ETOOBIG;
  if (d.H > 0 && !host_pinned) return ULA_EINVAL;
  void* ws = nullptr;
  int dev = -1;
  int rc = claim_static_workspace(&ws, &dev);
  if (rc) return rc;
  rc = init_impl(cfg, ws, host_pinned, stream, out, dev);   // releases the claim on failure
  return rc;
}

int ula_destroy(ula_ctx* ctx) {
  if (!ctx) return ULA_EINVAL;
  destroy_ctx(ctx);
  return ULA_OK;
}

// Host validation of an append batch (nothing changes on error).
static int validate_append(const ula_ctx* ctx, const GroupHost& gh, int32_t n, const int32_t* la_host) {
  const Dims& d = ctx->dims;
  for (int32_t i = 0; i < n; ++i)
    if (la_host[i] < 0 || la_host[i] >= d.N) return ULA_ERANGE;
  {
    std::vector<int32_t> sorted(la_host, la_host + n);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return ULA_EDUP;
  }
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t la = (uint32_t)la_host[i];
    if (gh.appended[la >> 6] >> (la & 63) & 1ull) return ULA_EDUP;
  }
  if (gh.n_appended + n > d.P + d.H) return ULA_EHOSTFULL;
  return ULA_OK;
}

static void note_appended(GroupHost& gh, int32_t n, const int32_t* la_host) {
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t la = (uint32_t)la_host[i];
    gh.appended[la >> 6] |= 1ull << (la & 63);
  }
  gh.n_appended += n;
}

int ula_append(ula_ctx* ctx, int32_t group, int32_t n, const int32_t* la_host, const void* rows,
               int32_t rows_on_device, uint64_t stream) {
  if (!ctx) return ULA_EINVAL;
  if (ctx->poisoned) return ULA_ESTATE;
  if (group < 0 || group >= ctx->cfg.num_groups || n < 0) return ULA_EINVAL;
  if (n == 0) return ULA_OK;
  if (!la_host || !rows) return ULA_EINVAL;
  GroupHost& gh = ctx->groups[group];
  const Dims& d = ctx->dims;
  {
    const int rc = validate_append(ctx, gh, n, la_host);   // the whole batch first
    if (rc) return rc;
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const GroupDev& g = gh.d;
  // An append needs no wait for a pending eviction write-back: it writes only
  // free host slots, and no free host slot has one. A step's evicted rows go to
  // slots its misses vacated, which the evicted entries then occupy; a release
  // writes every staged row out before it frees a slot; and the host slot a miss
  // vacates when its victim was a free GPU slot receives no evicted row (nor had
  // one pending: its entry was in it during the previous step).
  // placement ring: the current bucket is that of the group's last enqueued step
  const int32_t cur = (int32_t)(gh.steps % d.B);
  const int32_t ring = d.placement == ULA_PLACE_RING ? 1 : 0;
  // Under ULA_PLACE_RING an append evicts GPU entries, so it waits for pending
  // gathers; otherwise it takes only free slots, which no gather reads.
  if (ring) {
    const int rc = wait_gathers(gh, s);
    if (rc) return rc;
  }
  if (n <= small_append_limit(d.policy) && n <= d.maxApp && rows_on_device) {
    // decode-time appends: one workgroup, addresses passed by value
    SmallAppend a{};
    a.n = n;
    a.ring = ring;
    a.cur = cur;
    std::memcpy(a.las, la_host, sizeof(int32_t) * n);
    HIP_TRY(launch_append_small(g, a, static_cast<const uint8_t*>(rows), s));
  } else if (ctx->static_dev >= 0) {
    // a context without pinned staging buffers: chunks whose addresses go by
    // value; host rows are copied in and waited for before the next chunk
    const int32_t chunk = (int32_t)std::min<int64_t>(kSmallAppend, d.maxApp);
    for (int32_t off = 0; off < n; off += chunk) {
      SmallAppend a{};
      a.n = std::min(chunk, n - off);
      a.ring = ring;
      a.cur = cur;
      std::memcpy(a.las, la_host + off, sizeof(int32_t) * a.n);
      const uint8_t* src = static_cast<const uint8_t*>(rows) + (size_t)off * d.slot_bytes;
      if (!rows_on_device) {
        HIP_TRY(hipMemcpyAsync(g.app_rows, src, (size_t)a.n * d.slot_bytes, hipMemcpyHostToDevice, s));
        HIP_TRY(hipStreamSynchronize(s));
        src = g.app_rows;
      }
      HIP_TRY(launch_append_small(g, a, src, s));
    }
  } else {
    for (int32_t off = 0; off < n; off += (int32_t)d.maxApp) {
      const int32_t cnt = (int32_t)std::min<int64_t>(n - off, d.maxApp);
      // addresses go through a pinned staging slot so the copy is truly asynchronous
      const int k = gh.stage_next;
      gh.stage_next = (k + 1) % kStageSlots;
      if (gh.stage_used[k]) HIP_TRY(hipEventSynchronize(gh.stage_ev[k]));
      gh.stage_used[k] = true;
      std::memcpy(gh.stage[k], la_host + off, sizeof(int32_t) * cnt);
      HIP_TRY(hipMemcpyAsync(g.app_la, gh.stage[k], sizeof(int32_t) * cnt, hipMemcpyHostToDevice, s));
      HIP_TRY(hipEventRecord(gh.stage_ev[k], s));
      const uint8_t* src = static_cast<const uint8_t*>(rows) + (size_t)off * d.slot_bytes;
      if (!rows_on_device) {
        HIP_TRY(hipMemcpyAsync(g.app_rows, src, (size_t)cnt * d.slot_bytes, hipMemcpyHostToDevice, s));
        src = g.app_rows;
      }
      if (ring) {
        const PlanArgs a = ring_append_plan(cnt, cur, (int32_t)d.B);
        HIP_TRY(launch_plan(g, a, s));
        HIP_TRY(launch_extract(g, kPlanAppendRing, a.dest, 2 * cnt, s));
        HIP_TRY(launch_place_ring(g, cnt, src, s));
        continue;
      }
      PlanArgs a{};
      a.mode = kPlanAppend;
      a.n = cnt;
      a.norder = 2;
      a.dest = kCold;
      a.order[0] = kFree;
      a.order[1] = kHostFreeId;
      HIP_TRY(launch_plan(g, a, s));
      HIP_TRY(launch_extract(g, kPlanAppend, kCold, cnt, s));
      HIP_TRY(launch_place(g, cnt, src, s));
    }
  }
  note_appended(gh, n, la_host);
  return ULA_OK;
}

int ula_release(ula_ctx* ctx, int32_t group, int32_t n, const int32_t* la_host, uint64_t stream) {
  if (!ctx) return ULA_EINVAL;
  if (ctx->poisoned) return ULA_ESTATE;
  if (group < 0 || group >= ctx->cfg.num_groups || n < 0) return ULA_EINVAL;
  if (n == 0) return ULA_OK;
  if (!la_host) return ULA_EINVAL;
  GroupHost& gh = ctx->groups[group];
  const Dims& d = ctx->dims;
  // validate the whole batch first; nothing changes on error
  for (int32_t i = 0; i < n; ++i)
    if (la_host[i] < 0 || la_host[i] >= d.N) return ULA_ERANGE;
  {
    std::vector<int32_t> sorted(la_host, la_host + n);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return ULA_EDUP;
  }
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t la = (uint32_t)la_host[i];
    if (!(gh.appended[la >> 6] >> (la & 63) & 1ull)) return ULA_ERANGE;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const GroupDev& g = gh.d;
  {   // a released GPU slot may be taken by the next append: pending gathers first
    const int rc = wait_gathers(gh, s);
    if (rc) return rc;
  }
  // A released host slot may be waiting for the last step's evicted row, and an
  // append may take it next: write the staged rows out first.
  if (gh.steps > 0 && gh.written_back != gh.steps) {
    HIP_TRY(launch_writeback(g, std::max<int32_t>(gh.last_pairs, 1), s));
    gh.written_back = gh.steps;
  }
  for (int32_t off = 0; off < n; off += (int32_t)d.maxApp) {
    const int32_t cnt = (int32_t)std::min<int64_t>(n - off, d.maxApp);
    if (ctx->static_dev >= 0) {
      // no pinned staging buffers: copy from the caller's memory and wait for it
      HIP_TRY(hipMemcpyAsync(g.app_la, la_host + off, sizeof(int32_t) * cnt, hipMemcpyHostToDevice, s));
      HIP_TRY(hipStreamSynchronize(s));
    } else {
      const int k = gh.stage_next;
      gh.stage_next = (k + 1) % kStageSlots;
      if (gh.stage_used[k]) HIP_TRY(hipEventSynchronize(gh.stage_ev[k]));
      gh.stage_used[k] = true;
      std::memcpy(gh.stage[k], la_host + off, sizeof(int32_t) * cnt);
      HIP_TRY(hipMemcpyAsync(g.app_la, gh.stage[k], sizeof(int32_t) * cnt, hipMemcpyHostToDevice, s));
      HIP_TRY(hipEventRecord(gh.stage_ev[k], s));
    }
    HIP_TRY(launch_release(g, cnt, s));
  }
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t la = (uint32_t)la_host[i];
    gh.appended[la >> 6] &= ~(1ull << (la & 63));
  }
  gh.n_appended -= n;
  gh.last_n = 0;   // the last step's resolved selection may name released entries
  return ULA_OK;
}

// The evicted rows a step stages reach the host in the group's next step (the
// write-back workgroups of its mark launch). Before the host reads rows, a
// stand-alone write-back puts the staged rows there too (those of the last
// step, or of an earlier one if a device error stopped the steps after it).
// The device is idle first, so the write-back runs on the null stream: the
// library never enqueues on a caller's stream outside a call that names it.
static int flush_writebacks(ula_ctx* ctx) {
  HIP_TRY(hipDeviceSynchronize());
  bool any = false;
  for (auto& gh : ctx->groups) {
    if (gh.steps == 0 || gh.written_back == gh.steps) continue;
    HIP_TRY(launch_writeback(gh.d, std::max<int32_t>(gh.last_pairs, 1), nullptr));
    gh.written_back = gh.steps;
    any = true;
  }
  if (any) HIP_TRY(hipDeviceSynchronize());
  return ULA_OK;
}

// Host checks of a step's arguments (nothing is enqueued on error).
static int validate_step(const ula_ctx* ctx, int32_t group, int32_t n_sets, int32_t k, const int32_t* sel_dev) {
  if (ctx->poisoned) return ULA_ESTATE;
  if (group < 0 || group >= ctx->cfg.num_groups) return ULA_EINVAL;
  if (n_sets < 0 || k < 0 || n_sets > ctx->cfg.max_sets || k > ctx->cfg.max_k) return ULA_EINVAL;
  if (n_sets * k > 0 && !sel_dev) return ULA_EINVAL;
  return ULA_OK;
}

// A validated step; `app` (nullable): a small append whose rows are in device
// memory, run in the step's first launch beside the tag pass.
static int step_impl(ula_ctx* ctx, int32_t group, int32_t n_sets, int32_t k, const int32_t* sel_dev,
                     uint64_t stream, const SmallAppend* app, const uint8_t* app_rows) {
  const int32_t n = n_sets * k;
  GroupHost& gh = ctx->groups[group];
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t t = gh.steps + 1;
  GroupDev g = gh.d;
  g.res = res_for(ctx, gh, t);   // the other buffer may still be read by the last step's gathers
  const int32_t cur = (int32_t)(t % ctx->dims.B);
  const bool tm = (ctx->timing & ULA_TIMING_STEP) != 0;
  const int32_t max_pairs = (int32_t)std::min<int64_t>(n, ctx->dims.maxU);
  // the previous step's evicted rows, unless a flush already wrote them out
  const int32_t wb_pairs = (gh.steps > 0 && gh.written_back != gh.steps) ? gh.last_pairs : 0;

  if (app && app->ring) {   // this append evicts GPU entries: pending gathers first
    const int rc = wait_gathers(gh, s);
    if (rc) return rc;
  }
  if (tm) HIP_TRY(hipEventRecord(gh.ev[0], s));
  if (app) HIP_TRY(launch_tag_append(g, *app, app_rows, sel_dev, n, (uint32_t)t, s));
  else HIP_TRY(launch_tag(g, sel_dev, n, (uint32_t)t, s));
  HIP_TRY(launch_compact(g, sel_dev, n, (uint32_t)t, s));
  if (tm) HIP_TRY(hipEventRecord(gh.ev[1], s));
  PlanArgs a{};
  a.mode = kPlanStep;
  a.dest = ring_id(cur);
  a.order[0] = kFree;
  a.order[1] = kCold;
  a.norder = 2;
  for (int j = 1; j < ctx->dims.B; ++j) a.order[a.norder++] = (int8_t)ring_id((cur + j) % ctx->dims.B);
  hipEvent_t lk0 = nullptr, lk1 = nullptr;   // the host-link launch's own events (ULA_TIMING_LINK)
  if (ctx->timing & ULA_TIMING_LINK) {
    int rc = next_timing_pair(ctx->link_t, &lk0, &lk1);
    if (rc) return rc;
  }
  // one host-link launch at a time across streams (see ula_ctx)
  if (!ctx->first_step_stream) ctx->first_step_stream = s;
  if (s != ctx->first_step_stream && !ctx->multi_stream) {
    ctx->multi_stream = true;
    HIP_TRY(hipEventCreateWithFlags(&ctx->link_ev, hipEventDisableTiming));
  }
  if (ctx->multi_stream && ctx->link_ev_stream && ctx->link_ev_stream != s)
    HIP_TRY(hipStreamWaitEvent(s, ctx->link_ev, 0));
  if (g.policy == ULA_POLICY_LRU) {
    // exact LRU: select passes over the whole pool (the first launch also carries
    // the host-link work), then the victim list in order
    HIP_TRY(launch_lru_select(g, (uint32_t)t, max_pairs, wb_pairs, s, lk0, lk1));
    HIP_TRY(launch_lru_order(g, (uint32_t)t, max_pairs, s));
  } else {
    // marking, victim plan and extraction, with the missed rows read in and the
    // previous step's evicted rows written out, in one launch
    HIP_TRY(launch_mark(g, (uint32_t)t, cur, a, max_pairs, wb_pairs, s, lk0, lk1));
  }
  if (ctx->multi_stream) {
    HIP_TRY(hipEventRecord(ctx->link_ev, s));
    ctx->link_ev_stream = s;
  }
  if (tm) HIP_TRY(hipEventRecord(gh.ev[2], s));
  {   // the swap moves rows out of GPU slots the last step's gathers may still read
    const int rc = wait_gathers(gh, s);
    if (rc) return rc;
  }
  HIP_TRY(launch_swap_commit(g, (uint32_t)t, max_pairs, s));
  if (tm) HIP_TRY(hipEventRecord(gh.ev[3], s));
  gh.steps = t;
  gh.last_n = n;
  gh.last_pairs = max_pairs;
  return ULA_OK;
}

int ula_step(ula_ctx* ctx, int32_t group, int32_t n_sets, int32_t k, const int32_t* sel_dev,
             uint64_t stream) {
  if (!ctx) return ULA_EINVAL;
  const int rc = validate_step(ctx, group, n_sets, k, sel_dev);
  if (rc) return rc;
  return step_impl(ctx, group, n_sets, k, sel_dev, stream, nullptr, nullptr);
}

int ula_append_step(ula_ctx* ctx, int32_t group, int32_t n_app, const int32_t* la_host, const void* rows,
                    int32_t rows_on_device, int32_t n_sets, int32_t k, const int32_t* sel_dev,
                    uint64_t stream) {
  if (!ctx) return ULA_EINVAL;
  {
    const int rc = validate_step(ctx, group, n_sets, k, sel_dev);
    if (rc) return rc;
  }
  if (n_app < 0) return ULA_EINVAL;
  if (n_app > 0) {
    if (!la_host || !rows) return ULA_EINVAL;
    const int rc = validate_append(ctx, ctx->groups[group], n_app, la_host);
    if (rc) return rc;
  }
  if (n_app > 0 && n_app <= small_append_limit(ctx->dims.policy) && n_app <= ctx->dims.maxApp &&
      rows_on_device) {
    SmallAppend a{};
    a.n = n_app;
    a.ring = ctx->dims.placement == ULA_PLACE_RING ? 1 : 0;
    a.cur = (int32_t)(ctx->groups[group].steps % ctx->dims.B);   // before the step advances it
    std::memcpy(a.las, la_host, sizeof(int32_t) * n_app);
    const int rc = step_impl(ctx, group, n_sets, k, sel_dev, stream, &a, static_cast<const uint8_t*>(rows));
    if (rc) return rc;
    note_appended(ctx->groups[group], n_app, la_host);
    return ULA_OK;
  }
  if (n_app > 0) {
    const int rc = ula_append(ctx, group, n_app, la_host, rows, rows_on_device, stream);
    if (rc) return rc;
  }
  return step_impl(ctx, group, n_sets, k, sel_dev, stream, nullptr, nullptr);
}

// Layers layer0 .. layer0 + nl - 1 of the selection, one launch.
static int gather_impl(ula_ctx* ctx, int32_t group, int32_t layer0, int32_t nl, int32_t n_sets, int32_t k,
                       const int32_t* sel_dev, void* out_dev, uint64_t stream) {
  if (!ctx) return ULA_EINVAL;
  if (ctx->poisoned) return ULA_ESTATE;
  if (group < 0 || group >= ctx->cfg.num_groups) return ULA_EINVAL;
  if (layer0 < 0 || nl < 1 || layer0 >= ctx->cfg.layers_per_group || nl > ctx->cfg.layers_per_group - layer0)
    return ULA_EINVAL;
  if (n_sets < 0 || k < 0 || n_sets > ctx->cfg.max_sets || k > ctx->cfg.max_k) return ULA_EINVAL;
  const int32_t n = n_sets * k;
  if (n > 0 && (!sel_dev || !out_dev)) return ULA_EINVAL;
  GroupHost& gh = ctx->groups[group];
  if (gh.steps == 0) return ULA_ENOTRESIDENT;
  hipEvent_t start = nullptr, stop = nullptr;
  if ((ctx->timing & ULA_TIMING_GATHER) && n > 0) {
    int rc = next_timing_pair(ctx->gather_t, &start, &stop);
    if (rc) return rc;
  }
  if (n == 0) return ULA_OK;
  GroupDev g = gh.d;
  g.res = res_for(ctx, gh, gh.steps);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(launch_gather(g, sel_dev, n, layer0, nl, static_cast<uint8_t*>(out_dev), (long long)gh.steps,
                        gh.last_n, s, start, stop));
  return note_gather(gh, s);
}

int ula_gather(ula_ctx* ctx, int32_t group, int32_t layer, int32_t n_sets, int32_t k,
               const int32_t* sel_dev, void* out_dev, uint64_t stream) {
  return gather_impl(ctx, group, layer, 1, n_sets, k, sel_dev, out_dev, stream);
}

int ula_gather_layers(ula_ctx* ctx, int32_t group, int32_t layer0, int32_t n_layers, int32_t n_sets,
                      int32_t k, const int32_t* sel_dev, void* out_dev, uint64_t stream) {
  return gather_impl(ctx, group, layer0, n_layers, n_sets, k, sel_dev, out_dev, stream);
}

static int read_counters(ula_ctx* ctx, std::vector<Counters>& out) {
  out.resize(ctx->cfg.num_groups);
  HIP_TRY(hipMemcpy(out.data(), ctx->ctrs, sizeof(Counters) * out.size(), hipMemcpyDeviceToHost));
  return ULA_OK;
}

static void fill_stats(const Counters& c, ula_step_stats* s) {
  s->unique = c.stats[0];
  s->hits = c.stats[1];
  s->misses = c.stats[2];
  s->evictions = c.stats[3];
  s->from_free = c.stats[4];
  s->invalid = c.stats[5];
}

int ula_sync(ula_ctx* ctx, uint64_t stream, ula_step_stats* per_group_out) {
  if (!ctx) return ULA_EINVAL;
  HIP_TRY(hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)));
  std::vector<Counters> c;
  int rc = read_counters(ctx, c);
  if (rc) return rc;
  int first = ULA_OK;
  for (size_t i = 0; i < c.size(); ++i) {
    if (per_group_out) fill_stats(c[i], &per_group_out[i]);
    const int code = c[i].status ? c[i].status : c[i].gstatus;
    if (code && first == ULA_OK) first = code;
  }
  if (first != ULA_OK) ctx->poisoned = first;
  return first;
}

int ula_export_state(ula_ctx* ctx, int32_t group, ula_state_host* out) {
  if (!ctx || !out) return ULA_EINVAL;
  if (group < 0 || group >= ctx->cfg.num_groups) return ULA_EINVAL;
  if (!out->map || !out->gown || !out->bitsets || (ctx->dims.H > 0 && !out->hown)) return ULA_EINVAL;
  // the exported fields do not depend on the host pool's rows, so staged
  // evicted rows stay staged (the group's next step writes them out as usual)
  HIP_TRY(hipDeviceSynchronize());
  const GroupDev& g = ctx->groups[group].d;
  const Dims& d = ctx->dims;
  HIP_TRY(hipMemcpy(out->map, g.map, 4 * d.N, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(out->gown, g.gown, 4 * d.P, hipMemcpyDeviceToHost));
  if (d.H > 0) HIP_TRY(hipMemcpy(out->hown, g.hown, 4 * d.H, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(out->bitsets, g.bm, 4 * d.NB * d.W, hipMemcpyDeviceToHost));
  if (d.policy == ULA_POLICY_LRU) {
    // exact LRU keeps only the free set; its timestamps, in the textbook form:
    // an occupied slot that no step stamped counts as s - P
    std::fill(out->bitsets + d.W, out->bitsets + d.NB * d.W, 0u);
    if (out->stamps) {
      HIP_TRY(hipMemcpy(out->stamps, g.lru_ts, 4 * d.P, hipMemcpyDeviceToHost));
      for (int64_t s = 0; s < d.P; ++s)
        if (out->gown[s] != -1 && out->stamps[s] < 1) out->stamps[s] = (int32_t)(s - d.P);
    }
  }
  Counters c;
  HIP_TRY(hipMemcpy(&c, g.ctr, sizeof(Counters), hipMemcpyDeviceToHost));
  out->flag = c.flag & ~kFlagFailed;   // the last completed step
  // derived, not read back: the ring advances once per step, so after step t the
  // current bucket is t mod B (the bucket bitsets show where the step's entries went)
  out->cur = (int32_t)(out->flag % d.B);
  fill_stats(c, &out->last);
  return ULA_OK;
}

int ula_read_rows(ula_ctx* ctx, int32_t group, int32_t n, const int32_t* la_host, void* out_host) {
  if (!ctx || n < 0) return ULA_EINVAL;
  if (group < 0 || group >= ctx->cfg.num_groups) return ULA_EINVAL;
  if (n == 0) return ULA_OK;
  if (!la_host || !out_host) return ULA_EINVAL;
  const Dims& d = ctx->dims;
  for (int32_t i = 0; i < n; ++i)
    if (la_host[i] < 0 || la_host[i] >= d.N) return ULA_ERANGE;
  {
    int rc = flush_writebacks(ctx);
    if (rc) return rc;
  }
  const GroupDev& g = ctx->groups[group].d;
  // the requested entries' locations: the whole mapping table when they are a
  // large share of it, else their words one by one (the table may hold up to
  // 2^31 - 1 words, 8.6 GB)
  std::vector<uint32_t> where(n);
  if ((int64_t)n * 64 >= d.N) {
    std::vector<uint32_t> map(d.N);
    HIP_TRY(hipMemcpy(map.data(), g.map, 4 * d.N, hipMemcpyDeviceToHost));
    for (int32_t i = 0; i < n; ++i) where[i] = map[la_host[i]];
  } else {
    for (int32_t i = 0; i < n; ++i)
      HIP_TRY(hipMemcpy(&where[i], g.map + la_host[i], 4, hipMemcpyDeviceToHost));
  }
  for (int32_t i = 0; i < n; ++i)
    if (where[i] == kAbsent) return ULA_ERANGE;
  uint8_t* o = static_cast<uint8_t*>(out_host);
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t loc = where[i];
    if (loc & kHostBit) {
      HIP_TRY(hipMemcpy(o + (size_t)i * d.slot_bytes,
                        g.host + (size_t)(loc & ~kHostBit) * d.slot_bytes, d.slot_bytes,
                        hipMemcpyDefault));
    } else {
      HIP_TRY(hipMemcpy(o + (size_t)i * d.slot_bytes, g.pool + (size_t)loc * d.slot_bytes,
                        d.slot_bytes, hipMemcpyDeviceToHost));
    }
  }
  return ULA_OK;
}

int ula_flag_address(ula_ctx* ctx, int32_t group, void** dev_ptr) {
  if (!ctx || !dev_ptr) return ULA_EINVAL;
  if (group < 0 || group >= ctx->cfg.num_groups) return ULA_EINVAL;
  *dev_ptr = &ctx->groups[group].d.ctr->flag;
  return ULA_OK;
}

int ula_set_timing(ula_ctx* ctx, int32_t flags) {
  if (!ctx || (flags & ~(ULA_TIMING_STEP | ULA_TIMING_GATHER | ULA_TIMING_LINK))) return ULA_EINVAL;
  if (flags & ULA_TIMING_STEP)   // a static-workspace context creates its step events here
    for (auto& gh : ctx->groups)
      for (auto& e : gh.ev)
        if (!e) HIP_TRY(hipEventCreate(&e));
  ctx->timing = flags;
  return ULA_OK;
}

int ula_read_gather_timing(ula_ctx* ctx, double* kernel_ms, int64_t* launches) {
  if (!ctx || !kernel_ms || !launches) return ULA_EINVAL;
  return drain_timing(ctx->gather_t, kernel_ms, launches);
}

int ula_read_link_timing(ula_ctx* ctx, double* kernel_ms, int64_t* launches) {
  if (!ctx || !kernel_ms || !launches) return ULA_EINVAL;
  return drain_timing(ctx->link_t, kernel_ms, launches);
}

int ula_read_timing(ula_ctx* ctx, int32_t group, float* ms_out3) {
  if (!ctx || !ms_out3) return ULA_EINVAL;
  if (group < 0 || group >= ctx->cfg.num_groups) return ULA_EINVAL;
  GroupHost& gh = ctx->groups[group];
  if (!gh.ev[3]) return ULA_EINVAL;   // step timing never switched on
  HIP_TRY(hipEventSynchronize(gh.ev[3]));
  for (int i = 0; i < 3; ++i) HIP_TRY(hipEventElapsedTime(&ms_out3[i], gh.ev[i], gh.ev[i + 1]));
  return ULA_OK;
}

}  // extern "C"
