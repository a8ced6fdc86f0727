// Ring advance with fold, and ordered selection of set bits (victims, free slots).
//
// Policy (UlaCache summary, paper-daily.com, section 3): a step moves the ring
// index on by one; the bucket it lands on still holds slots from B steps ago,
// which are relabelled cold (no data moves). Victims come from the free set,
// then cold, then the other ring buckets in age order, and the bucket of the
// running step is exempt. A bucket is a bit per GPU slot; counts per span above
// the bits let the selection jump over spans with no set bit.
//
// Summary hierarchy used here:
//   level 0  the bucket bitmaps, one bit per slot (canonical state)
//   level 1  tcnt: set bits per 2048-slot span (64 words), kept exact by every
//            kernel that moves a slot; a span with count 0 is the pages'
//            "empty segment" and is never read
//   level 2  per 64 spans, a bitmap of non-empty spans, built in LDS by the
//            plan kernel from level 1 with one wavefront ballot; popcounts over
//            it give each contributing span its work-item index, so empty spans
//            never produce work.
//
//   mark     fold and hit marking in one word-parallel pass over the spans that
//            have hits or survivors to fold (see the kernel); its last
//            workgroup then runs the plan. The same launch carries the
//            host-link work of the miss path (missed rows in, the previous
//            step's evicted rows out), so the transfers overlap the marking and
//            the planning.
//   plan     one workgroup (the last one of the mark kernel for a step, a
//            kernel of its own for an append): the quota of each bucket in eviction order (from
//            the exact bucket counts), then, per bucket with a quota, its
//            level-1 counts 1024 spans at a time, scanned across the workgroup to
//            give each contributing span its output offset and how many bits it
//            gives. Emits one work item per contributing span.
//   extract  one wavefront per work item: 64 lanes load the span's 64 words,
//            an exclusive prefix of their popcounts ranks every set bit, and
//            each lane writes the slots of its lowest set bits that fall below
//            the span's quota, in ascending slot order. The taken bits leave
//            their bucket and join the destination bucket.
#include <hip/hip_ext.h>
#include <algorithm>

#include "miss_path.h"
#include "tag_part.h"

namespace ula {

// Selection plan (one 1024-thread workgroup). STEP mode: m = misses of the
// step, sources in eviction order, destination ring[cur]. APPEND mode: m = n,
// sources [free, free host slots]: the first min(n, free GPU slots) entries take
// free GPU slots (joining cold), the rest free host slots. APPEND_RING mode:
// the step's sources (free, cold, ring oldest to newest) give the first
// q = min(n, available) slots, which join the current bucket; the free host
// source then gives n - q_free slots, right after them in the output: one for
// each entry displaced from an occupied slot, then one for each of the n - q
// entries left over. The GPU slots taken and the free ones among them go to
// the counter block (app_q, app_qfree) and, if s_q is given (LDS), to s_q[0..1].
// Work items go to `items`; returns their number (in every thread). pre_avail /
// pre_hint (nullable, LDS): the order's bucket counts and the free sets' span
// hints (GPU, host), already loaded by the caller.
__device__ int plan_body(const GroupDev& g, const PlanArgs& a, int* scratch,
                         unsigned long long* s_nonempty, SelItem* items,
                         const int* pre_avail = nullptr, const int* pre_hint = nullptr,
                         int* s_q = nullptr) {
  Counters* c = g.ctr;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  if (a.mode == kPlanStep) {
    // bucket counts: add the mark kernel's per-workgroup deltas
    for (int i = tid; i < g.NB; i += blockDim.x) {
      int s = 0;
      for (int b = 0; b < kMarkBlocks; ++b) s += g.partial[b * kMaxBuckets + i];
      c->bcnt[i] += s;
    }
    __syncthreads();
  }
  const int m = (a.mode == kPlanStep) ? c->n_miss : a.n;
  const bool ring = a.mode == kPlanAppendRing;
  int off = 0;       // output entries planned so far
  int nitems = 0;    // work items written so far
  int q_free = 0;
  int q_gpu = 0;     // GPU slots taken (APPEND_RING)
  for (int j = 0; j < a.norder && (off < m || ring); ++j) {
    const int id = a.order[j];
    const bool ring_host = ring && id == kHostFreeId;
    if (ring_host) q_gpu = off;
    const int want = ring_host ? a.n - q_free : m - off;
    if (want <= 0) continue;
    const int avail = pre_avail ? pre_avail[j] : *bucket_count(g, id);
    const int q = min(want, avail);
    if (q <= 0) continue;
    const uint32_t* tc = bucket_tcnt(g, id);
    const int T = bucket_ntiles(g, id);
    // the free sets start at their hint: every span before it is empty
    int32_t* hint = id == kFree ? &c->free_lo : (id == kHostFreeId ? &c->hfree_lo : nullptr);
    const int start = hint ? (pre_hint ? pre_hint[id == kFree ? 0 : 1] : *hint) : 0;
    int pre = 0;   // set bits of this bucket in spans before the chunk
    for (int base = min(max(start, 0), T); base < T && pre < q; base += 1024) {
      const int tile = base + tid;
      const int cnt = tile < T ? (int)tc[tile] : 0;
      const unsigned long long ne = __ballot(cnt > 0);
      if (lane == 0) s_nonempty[wave] = ne;
      int total;
      const int ex = block_exclusive_sum<1024>(cnt, scratch, total);  // has barriers
      // A span contributes while the bits before it are below the quota. The
      // contributing spans are the first non-empty spans of the chunk, so a
      // span's item index is its rank among non-empty spans: popcounts of the
      // level-2 bitmap words before it plus its rank inside its own word.
      const bool emit = cnt > 0 && pre + ex < q;
      if (emit) {
        int rank = rank_below(ne);
        for (int w = 0; w < wave; ++w) rank += (int)__popcll(s_nonempty[w]);
        SelItem it;
        it.src = id;
        it.tile = tile;
        it.out_off = off + pre + ex;
        it.take = min(cnt, q - pre - ex);
        items[nitems + rank] = it;
        // the span where the quota is reached: everything before it is taken
        if (hint && pre + ex + cnt >= q) *hint = tile;
      }
      nitems += __syncthreads_count(emit);
      pre += total;
    }
    if (tid == 0) *bucket_count(g, id) -= q;
    if (id == kFree) q_free = q;
    off += q;
  }
  if (tid == 0) {
    c->n_items = nitems;
    if (a.mode == kPlanStep) {
      c->bcnt[a.dest] += m;
      c->stats[3] = m - q_free;   // evictions
      c->stats[4] = q_free;       // from free slots
    } else if (ring) {
      c->bcnt[a.dest] += q_gpu;
      c->app_q = q_gpu;
      c->app_qfree = q_free;
      if (s_q) {
        s_q[0] = q_gpu;
        s_q[1] = q_free;
      }
    } else {
      c->bcnt[a.dest] += q_free;
    }
  }
  return nitems;
}

__global__ __launch_bounds__(1024) void k_plan(GroupDev g, PlanArgs a) {
  __shared__ int scratch[1024 / kWave + 1];
  __shared__ unsigned long long s_nonempty[1024 / kWave];  // level-2 summary of a 1024-span chunk
  if (block_failed(g.ctr)) return;
  plan_body(g, a, scratch, s_nonempty, g.items);
}

// One wavefront takes the lowest `take` set bits of one span of one bitmap.
// STEP: taken GPU slots join ring[cur] (dest); the output list is the victims,
// and victims taken from the free bucket carry the top bit (their slot holds no
// row to evict). APPEND: taken GPU slots join cold (dest), taken host slots
// leave the free-host bitmap; the output list is the destinations (host slots
// carry the host bit). APPEND_RING: as STEP for the GPU slots (dest: the current
// bucket; free ones marked), then the host slots (host bit).
__device__ __forceinline__ void extract_item(const GroupDev& g, const SelItem it, int32_t mode,
                                             int32_t dest, uint32_t* out) {
  const int lane = lane_id();
  const bool host = it.src == kHostFreeId;
  const bool mark_free = (mode == kPlanStep || mode == kPlanAppendRing) && it.src == kFree;
  const uint32_t flag = (host || mark_free) ? kHostBit : 0u;
  uint32_t* words = bucket_words(g, it.src);
  const int w = it.tile * kTileWords + lane;
  const uint32_t x = w < bucket_nwords(g, it.src) ? words[w] : 0u;
  const int cnt = __popc(x);
  const int ex = wave_inclusive_sum(cnt) - cnt;
  int mine = it.take - ex;                    // lowest set bits this lane gives
  mine = mine < 0 ? 0 : (mine > cnt ? cnt : mine);
  uint32_t y = x, taken = 0;
  for (int r = 0; r < mine; ++r) {
    const uint32_t low = y & (0u - y);
    const uint32_t slot = (uint32_t)w * 32u + (uint32_t)(__ffs(y) - 1);
    y ^= low;
    taken |= low;
    out[it.out_off + ex + r] = flag | slot;
  }
  if (taken) {
    words[w] = x & ~taken;
    if (!host) atomicOr(&g.bm[(size_t)dest * g.W + w], taken);
  }
  if (lane == 0) {
    bucket_tcnt(g, it.src)[it.tile] -= (uint32_t)it.take;
    if (!host) atomicAdd(&g.tcnt[(size_t)dest * g.T + it.tile], (uint32_t)it.take);
  }
}

// Fold and hit marking, word-parallel and free of global atomics. One
// wavefront per 2048-slot span, lane = bitmap word. A span is visited only if
// it holds hits of this step (dirty == t) or survivors in ring[cur] to fold;
// the others are skipped from the summaries alone. For word w with hit mask
// hm (slots stamped t):
//   cold     <- (cold | ring[cur]) & ~hm      fold, then hits leave cold
//   ring[cur] <- hm                           hits join the new current bucket
//   ring[b]  <- ring[b] & ~hm  (b != cur)     hits leave older ring buckets
// Hits are never free slots. Span counts are recomputed by wavefront popcount
// sums; bucket-count changes go to per-workgroup partials, which the last
// workgroup adds up when it plans the step's victims.
//
// The same launch carries the rest of the step's selection and the host-link
// work of the miss path in extra workgroups:
//   - `pf` prefetch workgroups read the step's missed rows into HBM (victims
//     are not known yet; the swap kernel moves them into the victim slots over
//     HBM);
//   - `wbb` write-back workgroups write the previous step's evicted rows out,
//     when wb_step names that step; both link directions then run concurrently,
//     and only beside this launch's own marking and planning;
//   - `nh` extraction workgroups wait for the victim plan, then take one work
//     item per wavefront, together with the planning workgroup.
// Roles follow the order in which workgroups start (a ticket), so every
// workgroup that waits started after all the workgroups it waits for, which
// are resident and never wait themselves.
__device__ __forceinline__ void extract_part(const GroupDev& g, int32_t dest, int part, int nparts) {
  const int nitems = g.ctr->n_items;
  const int wpb = blockDim.x / kWave;
  for (int i = part * wpb + threadIdx.x / kWave; i < nitems; i += nparts * wpb)
    extract_item(g, g.items[i], kPlanStep, dest, g.victims);
}

constexpr int kPlanWaitLimit = 1 << 20;

__global__ __launch_bounds__(1024) void k_mark(GroupDev g, uint32_t t, int32_t cur, PlanArgs a,
                                               FastDiv per_slot, int32_t pf, int32_t wbb, int32_t nh,
                                               uint32_t wb_step) {
  __shared__ int s_delta[kMaxBuckets];
  __shared__ int s_last, s_role, s_fail, s_status, s_nmiss, s_wbn;
  __shared__ uint32_t s_wbstep;
  __shared__ int scratch[1024 / kWave + 1];
  __shared__ unsigned long long s_nonempty[1024 / kWave];
  // the error status, the role ticket and the link roles' counts in one round
  // trip (a workgroup that then stops has taken a role; the step has failed, so
  // no role is waited for)
  if (threadIdx.x == 0) {
    s_status = status_of(g.ctr);
    s_fail = 0;
  } else if (threadIdx.x == kWave) {
    s_role = atomicAdd(&g.ctr->mark_role, 1);
  } else if (threadIdx.x == 2 * kWave) {
    s_nmiss = g.ctr->n_miss;
  } else if (threadIdx.x == 3 * kWave) {
    s_wbstep = g.ctr->wb_step;
  } else if (threadIdx.x == 4 * kWave) {
    s_wbn = g.ctr->wb_n;
  }
  __syncthreads();
  if (s_status) return;
  const int role = s_role;
  if (role < 0 || role >= (int)gridDim.x) {   // a corrupt ticket: never index with it
    if (threadIdx.x == 0) latch(g.ctr, ULA_ESTATE);
    return;
  }
  if (role >= kMarkBlocks + pf + wbb) {
    // extraction: wait until the planning workgroup publishes the plan
    if (threadIdx.x == 0) {
      int spins = 0;
      while (__hip_atomic_load(&g.ctr->plan_done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != t) {
        if (++spins > kPlanWaitLimit || status_of(g.ctr)) {
          s_fail = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (s_fail && !status_of(g.ctr)) latch(g.ctr, ULA_ESTATE);   // a wait that never ended
    }
    __syncthreads();
    if (!s_fail) extract_part(g, a.dest, role - (kMarkBlocks + pf + wbb), nh + 1);
    return;
  }
  if (role >= kMarkBlocks) {
    link_part(g, s_nmiss, s_wbstep, s_wbn, wb_step, per_slot, role - kMarkBlocks, pf, wbb);
    return;
  }
  for (int i = threadIdx.x; i < kMaxBuckets; i += blockDim.x) s_delta[i] = 0;
  __syncthreads();
  const int lane = lane_id();
  const int nwaves = kMarkBlocks * (blockDim.x / kWave);
  const int rc = ring_id(cur);
  uint32_t* cold = g.bm + (size_t)kCold * g.W;
  uint32_t* ring = g.bm + (size_t)rc * g.W;
  uint32_t* ct = g.tcnt + (size_t)kCold * g.T;
  uint32_t* rt = g.tcnt + (size_t)rc * g.T;
  for (int tile = role * (blockDim.x / kWave) + threadIdx.x / kWave; tile < g.T; tile += nwaves) {
    const bool hits = g.dirty[tile] == (int32_t)t;
    const int fold_cnt = (int)rt[tile];
    if (!hits && fold_cnt == 0) continue;     // nothing to fold, no hit: skip the span
    const int w = tile * kTileWords + lane;
    const bool valid = w < g.W;
    uint32_t hm = 0;
    if (hits && valid) {
      const vec4u* sp = reinterpret_cast<const vec4u*>(g.stamp + (size_t)w * 32);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const vec4u s4 = sp[q];
        hm |= (uint32_t)(s4.x == t) << (4 * q) | (uint32_t)(s4.y == t) << (4 * q + 1) |
              (uint32_t)(s4.z == t) << (4 * q + 2) | (uint32_t)(s4.w == t) << (4 * q + 3);
      }
    }
    const uint32_t oc = valid ? cold[w] : 0u;
    const uint32_t orr = (valid && fold_cnt) ? ring[w] : 0u;
    const uint32_t nc = (oc | orr) & ~hm;
    if (valid) {
      if (nc != oc) cold[w] = nc;
      if (hm != orr) ring[w] = hm;
    }
    const int c_cold = wave_sum(__popc(nc));
    const int c_ring = wave_sum(__popc(hm));
    if (lane == 0) {
      const int old_cold = (int)ct[tile];
      ct[tile] = (uint32_t)c_cold;
      rt[tile] = (uint32_t)c_ring;
      atomicAdd(&s_delta[kCold], c_cold - old_cold);
      atomicAdd(&s_delta[rc], c_ring - fold_cnt);
    }
    if (hits) {
      // hits leave the other ring buckets; eight buckets' words in flight at once
      for (int b0 = 0; b0 < g.B; b0 += 8) {
        int ob[8];
        uint32_t x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int b = b0 + j;
          ob[j] = (b < g.B && b != cur) ? (int)g.tcnt[(size_t)ring_id(b) * g.T + tile] : 0;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          x[j] = (ob[j] && valid) ? g.bm[(size_t)ring_id(b0 + j) * g.W + w] : 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (!ob[j]) continue;               // empty span of this bucket (wave-uniform)
          const int id = ring_id(b0 + j);
          const uint32_t nx = x[j] & ~hm;
          if (valid && nx != x[j]) g.bm[(size_t)id * g.W + w] = nx;
          const int cb = wave_sum(__popc(nx));
          if (lane == 0 && cb != ob[j]) {
            g.tcnt[(size_t)id * g.T + tile] = (uint32_t)cb;
            atomicAdd(&s_delta[id], cb - ob[j]);
          }
        }
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kMaxBuckets; i += blockDim.x)
    g.partial[role * kMaxBuckets + i] = s_delta[i];
  // The last workgroup to finish plans the victims: one release per workgroup
  // before its ticket, the acquire-release ticket, and an acquire in the last
  // workgroup make every workgroup's bitmaps, span counts and partials visible.
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const int ticket = __hip_atomic_fetch_add(&g.ctr->done_mark, 1, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == kMarkBlocks - 1;
    if (ticket < 0 || ticket >= kMarkBlocks) latch(g.ctr, ULA_ESTATE);   // corrupt ticket: no plan
    if (s_last) {
      g.ctr->done_mark = 0;
      __threadfence();
    }
  }
  __syncthreads();
  if (!s_last) return;
  plan_body(g, a, scratch, s_nonempty, g.items);
  // publish the plan (items, counts) to the extraction workgroups, then join them
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    __hip_atomic_store(&g.ctr->plan_done, t, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
  extract_part(g, a.dest, nh, nh + 1);
}


__global__ __launch_bounds__(256) void k_extract(GroupDev g, int32_t mode, int32_t dest) {
  if (status_of(g.ctr)) return;
  const int nitems = g.ctr->n_items;
  const int nwaves = gridDim.x * (blockDim.x / kWave);
  uint32_t* out = (mode == kPlanStep) ? g.victims : g.app_dst;
  for (int i = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; i < nitems; i += nwaves)
    extract_item(g, g.items[i], mode, dest, out);
}

// A small append in one workgroup: plan, extraction and placement back to back
// (the same steps as the plan / extract / place kernels) with the work items and
// destinations in LDS, the addresses passed by value so that no copy precedes
// the launch, and the counters, span hints and first pieces of the rows loaded
// together before the plan: the chain of dependent memory accesses is the
// span counts, the bitmap words, then the stores. One 1024-lane workgroup.
__device__ void append_small_body(const GroupDev& g, const SmallAppend& a, const uint8_t* __restrict__ rows,
                                  FastDiv per_slot) {
  __shared__ int scratch[1024 / kWave + 1];
  __shared__ unsigned long long s_nonempty[1024 / kWave];
  // each item takes at least one output; under placement ring an entry can use
  // two outputs (its GPU slot and the host slot of the entry it displaces)
  __shared__ SelItem s_items[2 * kSmallAppend];
  __shared__ uint32_t s_dst[2 * kSmallAppend];
  __shared__ int s_status, s_avail[2], s_hint[2], s_q[2];
  const int tid = threadIdx.x;
  if (tid == 0) s_status = status_of(g.ctr);
  else if (tid == kWave) s_avail[0] = g.ctr->bcnt[kFree];
  else if (tid == 2 * kWave) s_avail[1] = g.ctr->hfree;
  else if (tid == 3 * kWave) s_hint[0] = g.ctr->free_lo;
  else if (tid == 4 * kWave) s_hint[1] = g.ctr->hfree_lo;
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t total = (uint32_t)a.n * chunks;
  constexpr int kEarly = 2;   // pieces per lane loaded before the plan
  vec4u early[kEarly];
#pragma unroll
  for (int r = 0; r < kEarly; ++r) {
    const uint32_t idx = (uint32_t)tid + (uint32_t)r * 1024u;
    if (idx < total) {
      const uint32_t i = per_slot.div(idx);
      early[r] = reinterpret_cast<const vec4u*>(rows + (size_t)i * g.slot_bytes)[idx - i * chunks];
    }
  }
  __syncthreads();
  if (s_status) return;
  if (a.ring) {
    const PlanArgs p = ring_append_plan(a.n, a.cur, g.B);
    const int nitems = plan_body(g, p, scratch, s_nonempty, s_items, nullptr, s_hint, s_q);
    for (int i = tid / kWave; i < nitems; i += blockDim.x / kWave)
      extract_item(g, s_items[i], kPlanAppendRing, p.dest, s_dst);
  } else {
    PlanArgs p{};
    p.mode = kPlanAppend;
    p.n = a.n;
    p.norder = 2;
    p.dest = kCold;
    p.order[0] = kFree;
    p.order[1] = kHostFreeId;
    const int nitems = plan_body(g, p, scratch, s_nonempty, s_items, s_avail, s_hint);
    for (int i = tid / kWave; i < nitems; i += blockDim.x / kWave)
      extract_item(g, s_items[i], kPlanAppend, kCold, s_dst);
  }
  __syncthreads();
  auto place = [&](uint32_t idx, const vec4u v) {
    const uint32_t i = per_slot.div(idx);
    const uint32_t c = idx - i * chunks;
    if (a.ring) place_piece_ring(g, s_dst, s_q[0], s_q[1], i, c, a.las[i], v);
    else place_piece(g, s_dst[i], c, a.las[i], v);
  };
#pragma unroll
  for (int r = 0; r < kEarly; ++r) {
    const uint32_t idx = (uint32_t)tid + (uint32_t)r * 1024u;
    if (idx < total) place(idx, early[r]);
  }
  for (uint32_t idx = (uint32_t)tid + kEarly * 1024u; idx < total; idx += blockDim.x) {
    const uint32_t i = per_slot.div(idx);
    place(idx, reinterpret_cast<const vec4u*>(rows + (size_t)i * g.slot_bytes)[idx - i * chunks]);
  }
}

__global__ __launch_bounds__(1024) void k_append_small(GroupDev g, SmallAppend a,
                                                       const uint8_t* __restrict__ rows,
                                                       FastDiv per_slot) {
  append_small_body(g, a, rows, per_slot);
}

// A step's first launch with the step's small append beside it: the last
// workgroup appends, the others run the de-duplication tag pass, which reads
// only the selection; the two write disjoint data (tags, descriptors and the
// padding count; the mapping table, owners, buckets and rows of the appended
// entries). The compaction, in the next launch, sees both.
__global__ __launch_bounds__(1024) void k_tag_append(GroupDev g, SmallAppend a, const uint8_t* __restrict__ rows,
                                                     FastDiv per_slot, const int32_t* __restrict__ sel,
                                                     int32_t n, uint32_t t) {
  if ((int)blockIdx.x == (int)gridDim.x - 1) {
    append_small_body(g, a, rows, per_slot);
    return;
  }
  tag_entries(g, sel, n, t, blockIdx.x, gridDim.x - 1);
}

hipError_t launch_mark(const GroupDev& g, uint32_t t, int32_t cur, const PlanArgs& a,
                       int32_t max_pairs, int32_t wb_pairs, hipStream_t s, hipEvent_t start,
                       hipEvent_t stop) {
  // Prefetch workgroups: enough for the largest possible miss list, at most
  // kPrefetchBlocks (about 2 MB of host reads in flight). Write-back
  // workgroups: enough for the previous step's pairs, at most kWritebackBlocks
  // (about 1 MB of host writes in flight, which saturates the link). None of
  // either without a host pool, since a step then never misses.
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  auto blocks_for = [&](int32_t pairs, int cap) {
    const int64_t n = ((int64_t)pairs * chunks + 4 * 1024 - 1) / (4 * 1024);
    return (int)std::min<int64_t>(n, cap);
  };
  const int pf = g.H > 0 ? blocks_for(max_pairs, kPrefetchBlocks) : 0;
  const int wbb = g.H > 0 ? blocks_for(wb_pairs, kWritebackBlocks) : 0;
  const int nh = kExtractHelpers;
  if (start)
    hipExtLaunchKernelGGL(k_mark, dim3(kMarkBlocks + pf + wbb + nh), dim3(1024), 0, s, start, stop, 0, g, t,
                          cur, a, FastDiv(chunks), pf, wbb, nh, wbb > 0 ? t - 1u : 0u);
  else
    k_mark<<<kMarkBlocks + pf + wbb + nh, 1024, 0, s>>>(g, t, cur, a, FastDiv(chunks), pf, wbb, nh,
                                                        wbb > 0 ? t - 1u : 0u);
  return hipGetLastError();
}

hipError_t launch_plan(const GroupDev& g, const PlanArgs& a, hipStream_t s) {
  k_plan<<<1, 1024, 0, s>>>(g, a);
  return hipGetLastError();
}

hipError_t launch_append_small(const GroupDev& g, const SmallAppend& a, const uint8_t* rows,
                              hipStream_t s) {
  k_append_small<<<1, 1024, 0, s>>>(g, a, rows, FastDiv((uint32_t)g.slot_bytes / 16u));
  return hipGetLastError();
}

hipError_t launch_tag_append(const GroupDev& g, const SmallAppend& a, const uint8_t* rows,
                             const int32_t* sel, int32_t n, uint32_t t, hipStream_t s) {
  int blocks = (n + 1023) / 1024;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;   // also clears the look-back descriptors
  k_tag_append<<<blocks + 1, 1024, 0, s>>>(g, a, rows, FastDiv((uint32_t)g.slot_bytes / 16u), sel, n, t);
  return hipGetLastError();
}

hipError_t launch_extract(const GroupDev& g, int32_t mode, int32_t dest, int32_t max_items,
                          hipStream_t s) {
  int blocks = (max_items + 3) / 4;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  k_extract<<<blocks, 256, 0, s>>>(g, mode, dest);
  return hipGetLastError();
}

}  // namespace ula
