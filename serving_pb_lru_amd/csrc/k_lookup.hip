// Group lookup and de-duplication, then hit marking.
//
// UlaCache summary (paper-daily.com), section 2: the layers of a group share a
// selection, so its addresses are resolved and de-duplicated once for all of
// them; section 3: that work and the recency bookkeeping run across GPU threads. The selection is n = n_sets * k logical addresses, row-major; -1 is
// padding. The distinct addresses are kept in first-occurrence order.
//
//   tag      every in-range entry e stores key(t, e) = (t << 32) | ~e into
//            tag[la] with a 64-bit atomic max (tag_part.h), so after the pass
//            tag[la] holds the key of la's first occurrence in step t. An
//            address outside [0, N) is an error there; one never appended is
//            found by the compaction, which reads the mapping table anyway. A
//            step's small append may run in the same launch (k_select.hip).
//   compact  single pass with a decoupled look-back: workgroups take tickets in
//            start order; each classifies its 1024 entries (first occurrence on
//            the GPU = hit, on the host = miss, padding) with wavefront ballots,
//            publishes its counts, and adds up its predecessors' published
//            counts (or a predecessor's inclusive prefix) to get its output
//            offsets, so hits and misses land in first-occurrence order. A
//            predecessor always started earlier and publishes before it waits,
//            so every wait ends; waits are bounded all the same. Padding entries
//            are counted by the tag kernel. The last
//            workgroup knows the totals: more distinct entries than GPU slots is
//            a capacity error raised before any state changes, and a never
//            appended entry anywhere (its flag travels in the counts) leaves the
//            statistics as they were. Each hit is
//            stamped with the step and its span marked dirty; every entry is
//            resolved for the gathers.
#include "tag_part.h"

namespace ula {

__global__ __launch_bounds__(256) void k_tag(GroupDev g, const int32_t* __restrict__ sel,
                                             int32_t n, uint32_t t) {
  tag_entries(g, sel, n, t, blockIdx.x, gridDim.x);
}

// Look-back descriptor of a workgroup: status in bits 62-63 (0 = not yet, 1 =
// its own counts, 2 = inclusive prefix), bit 61 set if a never appended entry
// was seen (in the workgroup, or for a prefix anywhere up to it), misses in bits
// 31-60, hits in bits 0-30. The counts travel inside the descriptor, so relaxed
// atomics suffice.
constexpr unsigned long long kDescAgg = 1ull << 62;
constexpr unsigned long long kDescPre = 2ull << 62;
constexpr unsigned long long kDescStatus = 3ull << 62;
constexpr unsigned long long kDescBad = 1ull << 61;
constexpr uint32_t kCount31 = 0x7FFFFFFFu;
constexpr uint32_t kCount30 = 0x3FFFFFFFu;
constexpr int kSpinLimit = 1 << 16;

__device__ __forceinline__ unsigned long long desc_pack(unsigned long long status, bool bad, uint32_t h,
                                                        uint32_t m) {
  return status | (bad ? kDescBad : 0ull) | ((unsigned long long)m << 31) | (unsigned long long)h;
}

__global__ __launch_bounds__(kScanBlock) void k_compact(GroupDev g, const int32_t* __restrict__ sel,
                                                        int32_t n, uint32_t t, int32_t nblk) {
  constexpr int NW = kScanBlock / kWave;
  __shared__ int s_h[NW], s_m[NW];
  __shared__ int s_vid, s_fail, s_status, s_bad;
  __shared__ uint32_t s_eh, s_em;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  // the error status and the ticket in one round trip (a workgroup that then
  // stops has taken a ticket; the step has failed, so the order no longer matters)
  if (threadIdx.x == 0) {
    s_status = status_of(g.ctr);
    s_fail = 0;
    s_bad = 0;
  } else if (threadIdx.x == kWave) {
    s_vid = atomicAdd(&g.ctr->lb_ticket, 1);
  }
  __syncthreads();
  if (s_status) return;
  const int vid = s_vid;
  if (vid < 0 || vid >= nblk) {            // a corrupt ticket: never index with it
    if (threadIdx.x == 0) latch(g.ctr, ULA_ESTATE);
    return;
  }
  unsigned long long* desc = g.desc + (size_t)(t & 1u) * g.maxBlk;

  // classify and resolve every entry (repeats included) for the gathers
  const int e = vid * kScanBlock + threadIdx.x;
  int c = 0;
  int32_t la = -1;
  uint32_t loc = 0;
  unsigned long long stage_rec = ~0ull;
  if (e < n) {
    la = sel[e];
    if (la == -1) {
      c = 3;
      g.res[e] = make_uint2(0xFFFFFFFFu, kAbsent);
    } else if (la < 0 || la >= g.N || (loc = g.map[la]) == kAbsent) {
      // never appended (out-of-range addresses were stopped by the tag kernel)
      s_bad = 1;
      latch(g.ctr, ULA_ERANGE);
    } else {
      const unsigned long long key = g.tag[la];
      if (key == dedup_key(t, (uint32_t)e)) {
        c = (loc & kHostBit) ? 2 : 1;
        g.res[e] = make_uint2((uint32_t)la, c == 1 ? loc : kAbsent);   // a miss's slot comes at commit
        // a miss's staging record, loaded now so that it arrives during the look-back
        if (c == 2) stage_rec = g.hs_stage[loc & ~kHostBit];
      } else {
        // a repeat: a hit resolves to its slot, a missed entry to its first occurrence
        const uint32_t first = ~(uint32_t)key;
        g.res[e] = make_uint2((uint32_t)la, (loc & kHostBit) ? (kHostBit | first) : loc);
      }
    }
  }
  const unsigned long long bh = __ballot(c == 1), bm = __ballot(c == 2);
  if (lane == 0) {
    s_h[wave] = __popcll(bh);
    s_m[wave] = __popcll(bm);
  }
  __syncthreads();

  // publish this workgroup's counts, then look back for its offsets (wave 0)
  if (wave == 0) {
    const bool bad = s_bad != 0;
    uint32_t ah = 0, am = 0;
    for (int w = 0; w < NW; ++w) {
      ah += s_h[w];
      am += s_m[w];
    }
    if (lane == 0)
      __hip_atomic_store(&desc[vid], desc_pack(vid == 0 ? kDescPre : kDescAgg, bad, ah, am), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    uint32_t eh = 0, em = 0;
    bool ebad = false;   // a never appended entry before this workgroup
    int j = vid - 1;     // predecessor examined by lane 0
    int spins = 0;
    while (j >= 0) {
      const int k = j - lane;
      const unsigned long long d =
          k >= 0 ? __hip_atomic_load(&desc[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kDescPre;
      const unsigned long long st = d & kDescStatus;
      const unsigned long long pre = __ballot(st == kDescPre);
      const unsigned long long zero = __ballot(st == 0ull);
      // lanes up to the nearest inclusive prefix must all have published
      const unsigned long long upto = pre ? ((pre & (0ull - pre)) << 1) - 1 : ~0ull;
      if (zero & upto) {
        if (++spins > kSpinLimit || status_of(g.ctr)) {
          if (lane == 0) s_fail = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        continue;
      }
      const bool take = (upto >> lane) & 1ull;
      int vh = take ? (int)(d & kCount31) : 0;
      int vm = take ? (int)((d >> 31) & kCount30) : 0;
      eh += (uint32_t)wave_sum(vh);
      em += (uint32_t)wave_sum(vm);
      ebad |= __ballot(take && (d & kDescBad) != 0ull) != 0ull;
      if (pre) break;
      j -= kWave;
    }
    if (lane == 0) {
      if (vid > 0 && !s_fail)
        __hip_atomic_store(&desc[vid], desc_pack(kDescPre, ebad || bad, eh + ah, em + am), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      s_eh = eh;
      s_em = em;
      if (vid == nblk - 1 && !s_fail) {
        // the last workgroup: every other one has published, so the totals are known
        Counters* cs = g.ctr;
        const int th = (int)(eh + ah), tm = (int)(em + am);
        const int tp = cs->pad_acc;   // counted by the tag kernel, which has completed
        const int u = th + tm;
        cs->lb_ticket = 0;
        cs->pad_acc = 0;
        if (ebad || bad) {
          // a never appended entry (already latched): the statistics stay as they were
        } else if (u > g.P) {
          latch(cs, ULA_ECAPACITY);   // before anything changes, statistics included
        } else {
          cs->n_hits = th;
          cs->n_miss = tm;
          cs->n_unique = u;
          cs->n_invalid = tp;
          cs->stats[0] = u;
          cs->stats[1] = th;
          cs->stats[2] = tm;
          cs->stats[3] = 0;
          cs->stats[4] = 0;
          cs->stats[5] = tp;
          cs->res_dup[t & 1u] = n - u - tp;
        }
      }
      if (s_fail && !status_of(g.ctr)) latch(g.ctr, ULA_ESTATE);   // a wait that never ended: give up cleanly
    }
  }
  __syncthreads();
  if (s_fail) return;
  if (c == 1) {
    int off = (int)s_eh;
    for (int w = 0; w < wave; ++w) off += s_h[w];
    const int pos = off + rank_below(bh);
    if (pos < g.maxU) g.hit_slots[pos] = loc;   // beyond the lists only on a capacity error
    // the bucket move itself is done word-parallel by the mark kernel, which
    // finds this step's hits by their stamp; every writer of a span's dirty
    // word writes the same value
    g.stamp[loc] = (int32_t)t;
    g.dirty[loc >> kTileShift] = (int32_t)t;
  } else if (c == 2) {
    int off = (int)s_em;
    for (int w = 0; w < wave; ++w) off += s_m[w];
    const int pos = off + rank_below(bm);
    if (pos < g.maxU) {
      const uint32_t h = loc & ~kHostBit;
      g.miss_la[pos] = la;
      g.miss_h[pos] = h;
      g.miss_e[pos] = e;
      // a row evicted by the previous step may still be on its way to the host:
      // read it from its staging copy instead
      const unsigned long long st = stage_rec;
      uint32_t from = kAbsent;
      if ((uint32_t)(st >> 32) == t - 1u) {
        from = (uint32_t)st;
        if (from >= (uint32_t)g.maxU) {   // corrupt staging record: no row to read
          latch(g.ctr, ULA_ESTATE);
          from = kAbsent;
        }
      }
      g.miss_stage[pos] = from;
    }
  }
}

hipError_t launch_tag(const GroupDev& g, const int32_t* sel, int32_t n, uint32_t t, hipStream_t s) {
  int blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;   // also clears the look-back descriptors
  k_tag<<<blocks, 256, 0, s>>>(g, sel, n, t);
  return hipGetLastError();
}

hipError_t launch_compact(const GroupDev& g, const int32_t* sel, int32_t n, uint32_t t, hipStream_t s) {
  int nblk = (n + kScanBlock - 1) / kScanBlock;
  if (nblk < 1) nblk = 1;   // one workgroup even for an empty selection: it publishes the (zero) totals
  k_compact<<<nblk, kScanBlock, 0, s>>>(g, sel, n, t, nblk);
  return hipGetLastError();
}

}  // namespace ula
