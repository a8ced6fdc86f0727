// Group lookup and de-duplication, then hit marking.
//
// UlaCache summary (paper-daily.com), section 2: layers sharing one sparse
// selection do the address lookup and de-duplication once per group; section 3:
// hit detection, recency update and de-duplication run in parallel on GPU
// threads. The selection is n = n_sets * k logical addresses, row-major; -1 is
// padding. The distinct addresses are kept in first-occurrence order.
//
//   tag      every valid entry e stores key(t, e) = (t << 32) | ~e into tag[la]
//            with a 64-bit atomic max, so after the kernel tag[la] holds the key
//            of la's first occurrence in step t (a smaller e gives a larger ~e;
//            tags of earlier steps have a smaller t and never match).
//   count    per block of 1024 entries: how many first occurrences are hits
//            (GPU-resident) and misses (host-resident), and how many are padding.
//   scan     one workgroup: exclusive offsets of the block counts; totals;
//            the capacity check (more distinct entries than GPU slots is an
//            error raised before any state changes).
//   compact  per block: wavefront ballot + mbcnt ranks the first occurrences
//            inside each wavefront, LDS adds the wavefront offsets, the block
//            offset comes from the scan: hits and misses land in first-occurrence
//            order. Each hit then leaves its bucket for the current ring bucket.
#include "device_util.h"

namespace ula {

__device__ __forceinline__ unsigned long long dedup_key(uint32_t t, uint32_t e) {
  return ((unsigned long long)t << 32) | (unsigned long long)(~e);
}

__global__ __launch_bounds__(256) void k_tag(GroupDev g, const int32_t* __restrict__ sel,
                                             int32_t n, uint32_t t) {
  if (status_of(g.ctr)) return;
  bool bad = false;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x) {
    int32_t la = sel[e];
    if (la == -1) continue;
    if (la < 0 || la >= g.N || g.map[la] == kAbsent) {
      bad = true;
      continue;
    }
    atomicMax(&g.tag[la], dedup_key(t, (uint32_t)e));
  }
  if (bad) latch(g.ctr, ULA_ERANGE);
}

// Classify entry e: 1 = first occurrence on the GPU, 2 = first occurrence on
// the host, 3 = padding, 0 = repeated. `loc` receives the mapping entry.
__device__ __forceinline__ int classify(const GroupDev& g, const int32_t* __restrict__ sel,
                                        int32_t n, int e, uint32_t t, int32_t& la,
                                        uint32_t& loc) {
  la = -1;
  loc = 0;
  if (e >= n) return 0;
  la = sel[e];
  if (la == -1) return 3;
  if (g.tag[la] != dedup_key(t, (uint32_t)e)) return 0;
  loc = g.map[la];
  return (loc & kHostBit) ? 2 : 1;
}

__global__ __launch_bounds__(kScanBlock) void k_count(GroupDev g, const int32_t* __restrict__ sel,
                                                      int32_t n, uint32_t t) {
  __shared__ int s[3][kScanBlock / kWave];
  if (block_failed(g.ctr)) return;
  const int e = blockIdx.x * kScanBlock + threadIdx.x;
  int32_t la;
  uint32_t loc;
  int c = classify(g, sel, n, e, t, la, loc);
  const int wave = threadIdx.x / kWave;
  unsigned long long bh = __ballot(c == 1), bm = __ballot(c == 2), bp = __ballot(c == 3);
  if (lane_id() == 0) {
    s[0][wave] = __popcll(bh);
    s[1][wave] = __popcll(bm);
    s[2][wave] = __popcll(bp);
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    int sum = 0;
    for (int w = 0; w < kScanBlock / kWave; ++w) sum += s[threadIdx.x][w];
    g.blk[3 * blockIdx.x + threadIdx.x] = (uint32_t)sum;
  }
}

// One workgroup turns the per-block counts into exclusive offsets (in place)
// and publishes the step's totals.
__global__ __launch_bounds__(1024) void k_scan(GroupDev g, int32_t nblk) {
  __shared__ int scratch[1024 / kWave + 1];
  if (block_failed(g.ctr)) return;
  int base_h = 0, base_m = 0, base_p = 0;
  for (int b0 = 0; b0 < nblk; b0 += 1024) {
    int b = b0 + threadIdx.x;
    int h = b < nblk ? (int)g.blk[3 * b] : 0;
    int m = b < nblk ? (int)g.blk[3 * b + 1] : 0;
    int p = b < nblk ? (int)g.blk[3 * b + 2] : 0;
    int th, tm, tp;
    int eh = block_exclusive_sum<1024>(h, scratch, th);
    int em = block_exclusive_sum<1024>(m, scratch, tm);
    block_exclusive_sum<1024>(p, scratch, tp);
    if (b < nblk) {
      g.blk[3 * b] = (uint32_t)(base_h + eh);
      g.blk[3 * b + 1] = (uint32_t)(base_m + em);
    }
    base_h += th;
    base_m += tm;
    base_p += tp;
  }
  if (threadIdx.x == 0) {
    Counters* c = g.ctr;
    int u = base_h + base_m;
    c->n_hits = base_h;
    c->n_miss = base_m;
    c->n_unique = u;
    c->n_invalid = base_p;
    c->stats[0] = u;
    c->stats[1] = base_h;
    c->stats[2] = base_m;
    c->stats[3] = 0;
    c->stats[4] = 0;
    c->stats[5] = base_p;
    if (u > g.P) latch(c, ULA_ECAPACITY);
  }
}

__global__ __launch_bounds__(kScanBlock) void k_compact(GroupDev g, const int32_t* __restrict__ sel,
                                                        int32_t n, uint32_t t, int32_t cur) {
  __shared__ int s_h[kScanBlock / kWave], s_m[kScanBlock / kWave];
  __shared__ int s_delta[kMaxBuckets];
  if (block_failed(g.ctr)) return;
  for (int i = threadIdx.x; i < g.NB; i += blockDim.x) s_delta[i] = 0;
  const int e = blockIdx.x * kScanBlock + threadIdx.x;
  int32_t la;
  uint32_t loc;
  int c = classify(g, sel, n, e, t, la, loc);
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  unsigned long long bh = __ballot(c == 1), bm = __ballot(c == 2);
  if (lane == 0) {
    s_h[wave] = __popcll(bh);
    s_m[wave] = __popcll(bm);
  }
  __syncthreads();
  if (c == 1 || c == 2) {
    int off = 0;
    if (c == 1) {
      for (int w = 0; w < wave; ++w) off += s_h[w];
      int pos = (int)g.blk[3 * blockIdx.x] + off + rank_below(bh);
      g.hit_slots[pos] = loc;
      // hit marking: the slot leaves its bucket and joins ring[cur]
      const uint32_t s = loc;
      const int32_t st = g.stamp[s];
      const int ob = (st > 0 && (int64_t)t - st < g.B) ? ring_id(st % g.B) : kCold;
      const int nb = ring_id(cur);
      const uint32_t bit = 1u << (s & 31);
      atomicAnd(&g.bm[(size_t)ob * g.W + (s >> 5)], ~bit);
      atomicOr(&g.bm[(size_t)nb * g.W + (s >> 5)], bit);
      atomicSub(&g.tcnt[(size_t)ob * g.T + (s >> kTileShift)], 1u);
      atomicAdd(&g.tcnt[(size_t)nb * g.T + (s >> kTileShift)], 1u);
      g.stamp[s] = (int32_t)t;
      atomicSub(&s_delta[ob], 1);
    } else {
      for (int w = 0; w < wave; ++w) off += s_m[w];
      int pos = (int)g.blk[3 * blockIdx.x + 1] + off + rank_below(bm);
      g.miss_la[pos] = la;
      g.miss_h[pos] = loc & ~kHostBit;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int nh = 0;
    for (int w = 0; w < kScanBlock / kWave; ++w) nh += s_h[w];
    s_delta[ring_id(cur)] += nh;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < g.NB; i += blockDim.x)
    if (s_delta[i]) atomicAdd(&g.ctr->bcnt[i], s_delta[i]);
}

hipError_t launch_tag(const GroupDev& g, const int32_t* sel, int32_t n, uint32_t t, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  k_tag<<<blocks, 256, 0, s>>>(g, sel, n, t);
  return hipGetLastError();
}

hipError_t launch_count(const GroupDev& g, const int32_t* sel, int32_t n, uint32_t t, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_count<<<(n + kScanBlock - 1) / kScanBlock, kScanBlock, 0, s>>>(g, sel, n, t);
  return hipGetLastError();
}

hipError_t launch_scan(const GroupDev& g, int32_t nblk, hipStream_t s) {
  k_scan<<<1, 1024, 0, s>>>(g, nblk);
  return hipGetLastError();
}

hipError_t launch_compact(const GroupDev& g, const int32_t* sel, int32_t n, uint32_t t,
                          int32_t cur, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_compact<<<(n + kScanBlock - 1) / kScanBlock, kScanBlock, 0, s>>>(g, sel, n, t, cur);
  return hipGetLastError();
}

}  // namespace ula
