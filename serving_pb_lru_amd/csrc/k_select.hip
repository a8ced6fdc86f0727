// Ring advance with fold, and ordered selection of set bits (victims, free slots).
//
// UlaCache summary (paper-daily.com), section 3: each round the current bucket
// advances one position and whatever is left in the bucket about to be reused
// moves to the cold bucket, by relabelling only; victims are free slots first,
// then the cold bucket, then ring buckets from oldest to newest, never the
// current bucket; each bucket is a bitmap with one bit per GPU slot, and
// summary levels above it let the selection skip empty segments.
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
//   fold     one wavefront per span of ring[cur] with a non-zero count: cold |=
//            ring[cur]; ring[cur] = 0; the span counts move along.
//   plan     one workgroup: the quota of each bucket in eviction order (from
//            the exact bucket counts), then, per bucket with a quota, its
//            level-1 counts 1024 spans at a time, scanned across the workgroup to
//            give each contributing span its output offset and how many bits it
//            gives. Emits one work item per contributing span.
//   extract  one wavefront per work item: 64 lanes load the span's 64 words,
//            an exclusive prefix of their popcounts ranks every set bit, and
//            each lane writes the slots of its lowest set bits that fall below
//            the span's quota, in ascending slot order. The taken bits leave
//            their bucket and join the destination bucket.
#include "device_util.h"

namespace ula {

__global__ __launch_bounds__(256) void k_fold(GroupDev g, int32_t cur) {
  if (status_of(g.ctr)) return;
  const int rb = ring_id(cur);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    g.ctr->bcnt[kCold] += g.ctr->bcnt[rb];
    g.ctr->bcnt[rb] = 0;
  }
  const int lane = lane_id();
  const int nwaves = gridDim.x * (blockDim.x / kWave);
  uint32_t* ring = g.bm + (size_t)rb * g.W;
  uint32_t* cold = g.bm + (size_t)kCold * g.W;
  uint32_t* rt = g.tcnt + (size_t)rb * g.T;
  uint32_t* ct = g.tcnt + (size_t)kCold * g.T;
  for (int tile = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; tile < g.T;
       tile += nwaves) {
    const uint32_t cnt = rt[tile];
    if (cnt == 0) continue;                 // empty span: skipped via the summary
    const int w = tile * kTileWords + lane;
    if (w < g.W) {
      const uint32_t r = ring[w];
      if (r) {
        cold[w] |= r;
        ring[w] = 0;
      }
    }
    if (lane == 0) {
      ct[tile] += cnt;
      rt[tile] = 0;
    }
  }
}

// Selection plan. STEP mode: m = misses of the step, sources in eviction order,
// destination ring[cur]. APPEND mode: m = n, sources [free, free host slots]:
// the first min(n, free GPU slots) entries take free GPU slots (joining cold),
// the rest free host slots.
__global__ __launch_bounds__(1024) void k_plan(GroupDev g, PlanArgs a) {
  __shared__ int scratch[1024 / kWave + 1];
  __shared__ unsigned long long s_nonempty[1024 / kWave];  // level-2 summary of a 1024-span chunk
  if (block_failed(g.ctr)) return;
  Counters* c = g.ctr;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int m = (a.mode == kPlanStep) ? c->n_miss : a.n;
  int off = 0;       // output entries planned so far
  int nitems = 0;    // work items written so far
  int q_free = 0;
  for (int j = 0; j < a.norder && off < m; ++j) {
    const int id = a.order[j];
    const int avail = *bucket_count(g, id);
    const int q = min(m - off, avail);
    if (q <= 0) continue;
    const uint32_t* tc = bucket_tcnt(g, id);
    const int T = bucket_ntiles(g, id);
    int pre = 0;   // set bits of this bucket in spans before the chunk
    for (int base = 0; base < T && pre < q; base += 1024) {
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
        g.items[nitems + rank] = it;
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
    } else {
      c->bcnt[a.dest] += q_free;
    }
  }
}

// STEP: taken GPU slots join ring[cur] (dest) with stamp t; the output list is
// the victims. APPEND: taken GPU slots join cold (dest) with stamp 0, taken
// host slots leave the free-host bitmap; the output list is the destinations
// (host slots carry the host bit).
__global__ __launch_bounds__(256) void k_extract(GroupDev g, int32_t mode, int32_t dest, uint32_t t) {
  if (status_of(g.ctr)) return;
  const int nitems = g.ctr->n_items;
  const int lane = lane_id();
  const int nwaves = gridDim.x * (blockDim.x / kWave);
  uint32_t* out = (mode == kPlanStep) ? g.victims : g.app_dst;
  const int32_t new_stamp = (mode == kPlanStep) ? (int32_t)t : 0;
  for (int i = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; i < nitems; i += nwaves) {
    const SelItem it = g.items[i];
    const bool host = it.src == kHostFreeId;
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
      out[it.out_off + ex + r] = host ? (kHostBit | slot) : slot;
      if (!host) g.stamp[slot] = new_stamp;
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
}

hipError_t launch_fold(const GroupDev& g, int32_t cur, hipStream_t s) {
  int blocks = (g.T + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  k_fold<<<blocks, 256, 0, s>>>(g, cur);
  return hipGetLastError();
}

hipError_t launch_plan(const GroupDev& g, const PlanArgs& a, hipStream_t s) {
  k_plan<<<1, 1024, 0, s>>>(g, a);
  return hipGetLastError();
}

hipError_t launch_extract(const GroupDev& g, int32_t mode, int32_t dest, uint32_t t,
                          int32_t max_items, hipStream_t s) {
  int blocks = (max_items + 3) / 4;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  k_extract<<<blocks, 256, 0, s>>>(g, mode, dest, t);
  return hipGetLastError();
}

}  // namespace ula
