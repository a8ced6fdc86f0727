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
//   compact  per block: the block's output offsets are the sums of the earlier
//            blocks' counts, the totals give the capacity check (more distinct
//            entries than GPU slots is an error raised before any state
//            changes); wavefront ballot + mbcnt ranks the first occurrences
//            inside each wavefront and LDS adds the wavefront offsets, so hits
//            and misses land in first-occurrence order. Each hit is stamped
//            with the step and its span marked dirty.
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

// Every workgroup adds up the counts of the workgroups before it (a few KB read
// from cache) to find its output offsets, and all of them add up the totals:
// they reach the same capacity verdict, so either every workgroup writes or
// none does. Workgroup 0 publishes the totals.
__global__ __launch_bounds__(kScanBlock) void k_compact(GroupDev g, const int32_t* __restrict__ sel,
                                                        int32_t n, uint32_t t, int32_t nblk) {
  __shared__ int s_h[kScanBlock / kWave], s_m[kScanBlock / kWave];
  __shared__ int s_tot[3][kScanBlock / kWave];
  __shared__ int s_base[3];
  if (block_failed(g.ctr)) return;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  {
    // counts of earlier workgroups (offsets) and of all workgroups (totals)
    int bh = 0, bmi = 0, ah = 0, am = 0, ap = 0;
    for (int b = threadIdx.x; b < nblk; b += kScanBlock) {
      const int h = (int)g.blk[3 * b], m = (int)g.blk[3 * b + 1], p = (int)g.blk[3 * b + 2];
      ah += h;
      am += m;
      ap += p;
      if (b < (int)blockIdx.x) {
        bh += h;
        bmi += m;
      }
    }
    bh = wave_sum(bh);
    bmi = wave_sum(bmi);
    ah = wave_sum(ah);
    am = wave_sum(am);
    ap = wave_sum(ap);
    if (lane == 0) {
      s_h[wave] = bh;
      s_m[wave] = bmi;
      s_tot[0][wave] = ah;
      s_tot[1][wave] = am;
      s_tot[2][wave] = ap;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int x[5] = {0, 0, 0, 0, 0};
      for (int w = 0; w < kScanBlock / kWave; ++w) {
        x[0] += s_h[w];
        x[1] += s_m[w];
        x[2] += s_tot[0][w];
        x[3] += s_tot[1][w];
        x[4] += s_tot[2][w];
      }
      s_base[0] = x[0];
      s_base[1] = x[1];
      const int u = x[2] + x[3];
      s_base[2] = u > g.P;
      if (blockIdx.x == 0 && u > g.P) {
        latch(g.ctr, ULA_ECAPACITY);   // before anything changes, statistics included
      } else if (blockIdx.x == 0) {
        Counters* c = g.ctr;
        c->n_hits = x[2];
        c->n_miss = x[3];
        c->n_unique = u;
        c->n_invalid = x[4];
        c->stats[0] = u;
        c->stats[1] = x[2];
        c->stats[2] = x[3];
        c->stats[3] = 0;
        c->stats[4] = 0;
        c->stats[5] = x[4];
      }
    }
    __syncthreads();
    if (s_base[2]) return;   // capacity error: nothing is written (uniform)
  }
  const int e = blockIdx.x * kScanBlock + threadIdx.x;
  // classify and resolve every entry (repeats included) for the gathers
  int c = 0;
  int32_t la = -1;
  uint32_t loc = 0;
  if (e < n) {
    la = sel[e];
    if (la == -1) {
      c = 3;
      g.res[e] = make_uint2(0xFFFFFFFFu, kAbsent);
    } else {
      const unsigned long long key = g.tag[la];
      loc = g.map[la];
      if (key == dedup_key(t, (uint32_t)e)) {
        c = (loc & kHostBit) ? 2 : 1;
        g.res[e] = make_uint2((uint32_t)la, c == 1 ? loc : kAbsent);   // a miss's slot comes at commit
      } else {
        // a repeat: a hit resolves to its slot, a missed entry to its first occurrence
        const uint32_t first = ~(uint32_t)key;
        g.res[e] = make_uint2((uint32_t)la, (loc & kHostBit) ? (kHostBit | first) : loc);
      }
    }
  }
  unsigned long long bh = __ballot(c == 1), bm = __ballot(c == 2);
  if (lane == 0) {
    s_h[wave] = __popcll(bh);
    s_m[wave] = __popcll(bm);
  }
  __syncthreads();
  if (c == 1) {
    int off = s_base[0];
    for (int w = 0; w < wave; ++w) off += s_h[w];
    g.hit_slots[off + rank_below(bh)] = loc;
    // the bucket move itself is done word-parallel by the mark kernel, which
    // finds this step's hits by their stamp; every writer of a span's dirty
    // word writes the same value
    g.stamp[loc] = (int32_t)t;
    g.dirty[loc >> kTileShift] = (int32_t)t;
  } else if (c == 2) {
    int off = s_base[1];
    for (int w = 0; w < wave; ++w) off += s_m[w];
    const int pos = off + rank_below(bm);
    g.miss_la[pos] = la;
    g.miss_h[pos] = loc & ~kHostBit;
    g.miss_e[pos] = e;
  }
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

hipError_t launch_compact(const GroupDev& g, const int32_t* sel, int32_t n, uint32_t t, hipStream_t s) {
  const int nblk = (n + kScanBlock - 1) / kScanBlock;
  // one workgroup even for an empty selection: it publishes the (zero) totals
  k_compact<<<nblk > 0 ? nblk : 1, kScanBlock, 0, s>>>(g, sel, n, t, nblk);
  return hipGetLastError();
}

}  // namespace ula
