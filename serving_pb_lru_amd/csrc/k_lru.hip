// Exact-LRU victim selection: one timestamp per GPU slot and a scan of the
// whole pool every step (the standard policy the pages compare PB-LRU against).
//
// UlaCache summary (paper-daily.com), section 3: textbook LRU stamps each slot
// with its last use and passes over the whole pool to pick victims, the cost
// PB-LRU's buckets avoid; section 4 compares the two (hit rate within 0.1 point,
// PB-LRU 1.5-2.3x faster to schedule at large batch, LRU faster when little is
// replaced). Lookup, pairing, data movement, commit and signal are shared with
// PB-LRU; only the choice and order of the victims differ.
//
// Victim order: free slots ascending, then occupied slots by (timestamp, slot),
// never a slot hit by the current step t. The commit gives the step's hits and
// loads timestamp t (so a failed step changes none); an appended slot keeps 0,
// standing for its textbook stamp s - P: older than every step and, among such
// slots, ordered by slot. So with the key
//   K(s) = 0 (free), excluded (hit this step), 1 (timestamp 0), timestamp + 1
// the order is (K, slot) ascending, exactly.
//
// Per step, with M misses:
//   select  up to three passes over every slot, each a histogram of the next key
//           digit (bits 21-31, 10-20, 0-9) among the slots whose higher digits
//           match the prefix found so far; the last workgroup of a pass finds the
//           digit where the running count reaches M. After the last, K* is the key
//           of the M-th victim, C the number of victims with a smaller key and
//           R = M - C the number taken from the slots with key K* (the lowest
//           slots first). No key exceeds the step number t (a timestamp is at
//           most t - 1), so the passes whose digits are zero for every key below
//           2^21 or 2^10 are skipped: before step 1024 a single pass decides.
//           The first pass's launch also carries the miss path's host-link
//           workgroups (prefetch and write-back), as the mark launch does under
//           PB-LRU.
//   count   one wavefront per 2048-slot span: how many slots have a key below K*
//           and how many have K*; the last workgroup turns both into offsets.
//   emit    one wavefront per span: slots with a key below K* go to a list in
//           slot order, the first R slots with key K* straight to their place in
//           the victim list (after the first C).
//   sort    a stable radix sort of that list by key (8-bit digits, as many passes
//           as the keys need) gives the first C victims in (K, slot) order.
#include <hip/hip_ext.h>
#include <algorithm>

#include "miss_path.h"

namespace ula {

constexpr uint32_t kExcludedKey = 0xFFFFFFFFu;
constexpr int kLruBins = 2048;

// Keys of the 32 slots of bitmap word w (slot 32 w + j in k[j]); slots >= P are
// excluded. The compaction marks this step's hits (stamp == t); the timestamps
// proper (lru_ts) change only at the commit. Both are padded to whole words;
// the owner array is read in the same 16-byte pieces (its region is padded to
// 64 entries).
__device__ __forceinline__ void word_keys(const GroupDev& g, int w, uint32_t t, uint32_t k[32]) {
  const vec4u* hp = reinterpret_cast<const vec4u*>(g.stamp + (size_t)w * 32);
  const vec4u* tp = reinterpret_cast<const vec4u*>(g.lru_ts + (size_t)w * 32);
  const vec4u* op = reinterpret_cast<const vec4u*>(g.gown + (size_t)w * 32);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const vec4u h4 = hp[q];
    const vec4u t4 = tp[q];
    const vec4u o4 = op[q];
    const uint32_t hm[4] = {h4.x, h4.y, h4.z, h4.w};
    const uint32_t ts[4] = {t4.x, t4.y, t4.z, t4.w};
    const uint32_t ow[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int32_t stamp = (int32_t)ts[j];
      uint32_t key;
      if ((int32_t)ow[j] == -1) key = 0u;
      else if ((int32_t)hm[j] == (int32_t)t) key = kExcludedKey;   // a hit of this step
      else key = stamp < 1 ? 1u : (uint32_t)stamp + 1u;
      k[4 * q + j] = key;
    }
  }
  const int base = w * 32;
#pragma unroll
  for (int j = 0; j < 32; ++j)
    if (base + j >= g.P) k[j] = kExcludedKey;
}

// Last workgroup of a select pass: find the digit where the running count of
// candidates reaches `need`, extend the prefix, count what lies below, and clear
// the histogram for the next pass. kLruThreads threads, consecutive bins each.
constexpr int kLruThreads = 512;    // select passes
constexpr int kSpanThreads = 256;   // count and emit (one wavefront per span)
constexpr int kBinsPerThread = kLruBins / kLruThreads;

__device__ void lru_find(const GroupDev& g, int nbins, int bits, int pass, int first, int* scratch) {
  __shared__ int s_bin, s_add;
  Counters* c = g.ctr;
  const int m = c->n_miss;
  const int below = pass == first ? 0 : c->lru_below;
  const int need = m - below;   // >= 1
  const int i0 = kBinsPerThread * threadIdx.x;
  int h[kBinsPerThread], sum = 0;
#pragma unroll
  for (int j = 0; j < kBinsPerThread; ++j) {
    h[j] = i0 + j < nbins ? (int)g.lru_hist[i0 + j] : 0;
    sum += h[j];
  }
  if (threadIdx.x == 0) s_bin = -1;
  int total;
  int pre = block_exclusive_sum<kLruThreads>(sum, scratch, total);   // has barriers
#pragma unroll
  for (int j = 0; j < kBinsPerThread; ++j) {
    if (pre < need && pre + h[j] >= need) {
      s_bin = i0 + j;
      s_add = pre;
    }
    pre += h[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBinsPerThread; ++j)
    if (i0 + j < nbins) g.lru_hist[i0 + j] = 0u;
  if (threadIdx.x == 0) {
    if (s_bin < 0) {
      latch(c, ULA_ESTATE);   // fewer candidates than misses: inconsistent state
    } else {
      const uint32_t prefix = pass == first ? (uint32_t)s_bin : (c->lru_prefix << bits) | (uint32_t)s_bin;
      const int nb = below + s_add;
      c->lru_prefix = prefix;
      c->lru_below = nb;
      if (pass == first) {
        const int ff = min(m, c->lru_nfree);
        c->stats[3] = m - ff;   // evictions
        c->stats[4] = ff;       // from free slots
        c->lru_nfree = 0;
      }
      if (pass == 2) {
        c->lru_kstar = prefix;
        c->lru_c = nb;
        c->lru_r = m - nb;
      }
    }
  }
}

// One select pass. Workgroups [0, nsel) histogram; in the first pass launched
// (`first`: the higher digits of every key are zero) the next pf workgroups
// prefetch the missed rows and the wbb after them write the previous step's
// evicted rows out (they wait for nothing).
__global__ __launch_bounds__(kLruThreads) void k_lru_pass(GroupDev g, uint32_t t, int32_t pass, int32_t first,
                                                   int32_t nsel,
                                                   FastDiv per_slot, int32_t pf, int32_t wbb,
                                                   uint32_t wb_step) {
  __shared__ uint32_t s_hist[kLruBins];
  __shared__ int s_free, s_last, s_status, s_nmiss, s_wbn;
  __shared__ uint32_t s_wbstep;
  __shared__ int scratch[kLruThreads / kWave + 1];
  // the error status and the counts every role needs, in one round trip
  if (threadIdx.x == 0) s_status = status_of(g.ctr);
  else if (threadIdx.x == kWave) s_nmiss = g.ctr->n_miss;
  else if (threadIdx.x == 2 * kWave) s_wbstep = g.ctr->wb_step;
  else if (threadIdx.x == 3 * kWave) s_wbn = g.ctr->wb_n;
  __syncthreads();
  if (s_status) return;
  if ((int)blockIdx.x >= nsel) {
    link_part(g, s_nmiss, s_wbstep, s_wbn, wb_step, per_slot, blockIdx.x - nsel, pf, wbb);
    return;
  }
  if (s_nmiss == 0) return;   // no victims to choose (uniform over the launch)
  const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
  const int bits = pass == 2 ? 10 : 11;
  const int nbins = 1 << bits;
  const uint32_t prefix = pass == first ? 0u : g.ctr->lru_prefix;
  for (int i = threadIdx.x; i < nbins; i += blockDim.x) s_hist[i] = 0u;
  if (threadIdx.x == 0) s_free = 0;
  __syncthreads();
  int nfree = 0;
  for (int w = blockIdx.x * blockDim.x + threadIdx.x; w < g.W; w += nsel * blockDim.x) {
    uint32_t k[32];
    word_keys(g, w, t, k);
    // runs of equal digits are added at once (keys of neighbouring slots agree
    // most of the time)
    int run_bin = -1, run = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t key = k[j];
      if (key == kExcludedKey) continue;
      nfree += key == 0u;
      if (pass > 0 && (key >> (shift + bits)) != prefix) continue;
      const int bin = (int)((key >> shift) & (uint32_t)(nbins - 1));
      if (bin != run_bin) {
        if (run) atomicAdd(&s_hist[run_bin], (uint32_t)run);
        run_bin = bin;
        run = 0;
      }
      ++run;
    }
    if (run) atomicAdd(&s_hist[run_bin], (uint32_t)run);
  }
  if (pass == first) {
    nfree = wave_sum(nfree);
    if (lane_id() == 0 && nfree) atomicAdd(&s_free, nfree);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nbins; i += blockDim.x)
    if (s_hist[i]) atomicAdd(&g.lru_hist[i], s_hist[i]);
  if (threadIdx.x == 0 && pass == first && s_free) atomicAdd(&g.ctr->lru_nfree, s_free);
  // the last workgroup to finish finds the digit (release per workgroup, then an
  // acquire-release ticket, as in the mark kernel)
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const int ticket = __hip_atomic_fetch_add(&g.ctr->lru_ticket, 1, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == nsel - 1;
    if (ticket < 0 || ticket >= nsel) latch(g.ctr, ULA_ESTATE);   // corrupt ticket
    if (s_last) {
      g.ctr->lru_ticket = 0;
      __threadfence();
    }
  }
  __syncthreads();
  if (!s_last) return;
  lru_find(g, nbins, bits, pass, first, scratch);
}

// Masks of the 32 slots of word w: below K*, and equal to K*; free slots among them.
__device__ __forceinline__ void word_masks(const GroupDev& g, int w, uint32_t t, uint32_t kstar,
                                           uint32_t& below, uint32_t& equal, uint32_t& freem,
                                           uint32_t k[32]) {
  below = equal = freem = 0u;
  if (w >= g.W) {
#pragma unroll
    for (int j = 0; j < 32; ++j) k[j] = kExcludedKey;
    return;
  }
  word_keys(g, w, t, k);
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    below |= (uint32_t)(k[j] < kstar) << j;
    equal |= (uint32_t)(k[j] == kstar) << j;
    freem |= (uint32_t)(k[j] == 0u) << j;
  }
}

// Exclusive prefix of span counts in place (one kSpanThreads-thread workgroup).
__device__ void spans_to_offsets(uint32_t* a, int n, int* scratch, int& total_out) {
  int carry = 0;
  for (int base = 0; base < n; base += kSpanThreads) {
    const int i = base + threadIdx.x;
    const int v = i < n ? (int)a[i] : 0;
    int total;
    const int ex = block_exclusive_sum<kSpanThreads>(v, scratch, total);
    if (i < n) a[i] = (uint32_t)(carry + ex);
    carry += total;
  }
  total_out = carry;
}

__global__ __launch_bounds__(kSpanThreads) void k_lru_count(GroupDev g, uint32_t t) {
  __shared__ int s_last;
  __shared__ int scratch[kSpanThreads / kWave + 1];
  if (block_failed(g.ctr)) return;
  if (g.ctr->n_miss == 0) return;
  const uint32_t kstar = g.ctr->lru_kstar;
  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  for (int tile = blockIdx.x * wpb + threadIdx.x / kWave; tile < g.T; tile += gridDim.x * wpb) {
    uint32_t below, equal, freem, k[32];
    word_masks(g, tile * kTileWords + lane, t, kstar, below, equal, freem, k);
    const int ca = wave_sum(__popc(below));
    const int cb = wave_sum(__popc(equal));
    if (lane == 0) {
      g.span_a[tile] = (uint32_t)ca;
      g.span_b[tile] = (uint32_t)cb;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const int ticket = __hip_atomic_fetch_add(&g.ctr->lru_ticket, 1, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == (int)gridDim.x - 1;
    if (ticket < 0 || ticket >= (int)gridDim.x) latch(g.ctr, ULA_ESTATE);
    if (s_last) {
      g.ctr->lru_ticket = 0;
      __threadfence();
    }
  }
  __syncthreads();
  if (!s_last) return;
  int ta, tb;
  spans_to_offsets(g.span_a, g.T, scratch, ta);
  spans_to_offsets(g.span_b, g.T, scratch, tb);
  if (threadIdx.x == 0 && (ta != g.ctr->lru_c || tb < g.ctr->lru_r))
    latch(g.ctr, ULA_ESTATE);   // the counts disagree with the select passes
}

__global__ __launch_bounds__(kSpanThreads) void k_lru_emit(GroupDev g, uint32_t t) {
  if (block_failed(g.ctr)) return;
  if (g.ctr->n_miss == 0) return;
  const uint32_t kstar = g.ctr->lru_kstar;
  const int C = g.ctr->lru_c, R = g.ctr->lru_r;
  const bool direct = kstar <= 1u;   // every key below K* is 0 (free): slot order is final
  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  uint32_t* fwords = g.bm + (size_t)kFree * g.W;
  for (int tile = blockIdx.x * wpb + threadIdx.x / kWave; tile < g.T; tile += gridDim.x * wpb) {
    const int w = tile * kTileWords + lane;
    uint32_t below, equal, freem, k[32];
    word_masks(g, w, t, kstar, below, equal, freem, k);
    const int na = __popc(below), nb = __popc(equal);
    int ra = (int)g.span_a[tile] + wave_inclusive_sum(na) - na;
    int rb = (int)g.span_b[tile] + wave_inclusive_sum(nb) - nb;
    uint32_t taken_free = below & freem;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t bit = 1u << j;
      const uint32_t slot = (uint32_t)w * 32u + (uint32_t)j;
      if (below & bit) {
        if (direct) {
          g.victims[ra] = kHostBit | slot;
        } else {
          g.sort_key[0][ra] = k[j];
          g.sort_slot[0][ra] = slot;
        }
        ++ra;
      } else if (equal & bit) {
        if (rb < R) {
          g.victims[C + rb] = (kstar == 0u ? kHostBit : 0u) | slot;
          if (kstar == 0u) taken_free |= bit;
        }
        ++rb;
      }
    }
    // victims taken from the free set leave it
    if (taken_free) atomicAnd(&fwords[w], ~taken_free);
    const int nf = wave_sum(__popc(taken_free));
    if (lane == 0 && nf) {
      atomicSub(&g.tcnt[(size_t)kFree * g.T + tile], (uint32_t)nf);
      atomicSub(&g.ctr->bcnt[kFree], nf);
    }
  }
}

// Stable radix sort of the first C victims by key, 8 bits per pass. Pass p is
// active when the keys below K* need more than 8 p bits; the last active pass
// writes the victim list. Blocks of 1024 entries.
__device__ __forceinline__ int sort_passes(uint32_t kstar) {
  if (kstar <= 1u) return 0;   // written directly by the emit kernel
  const int nbits = 32 - __clz((int)(kstar - 1u));
  return (nbits + 7) / 8;
}

__global__ __launch_bounds__(1024) void k_rs_count(GroupDev g, int32_t pass) {
  __shared__ uint32_t s_cnt[256];
  __shared__ int s_last;
  __shared__ int scratch[1024 / kWave + 1];
  if (block_failed(g.ctr)) return;
  if (g.ctr->n_miss == 0) return;
  const int C = g.ctr->lru_c;
  if (pass >= sort_passes(g.ctr->lru_kstar) || C == 0) return;   // uniform over the launch
  const int nblk = (C + 1023) / 1024;
  const int b = blockIdx.x;
  const uint32_t* key = g.sort_key[pass & 1];
  if (threadIdx.x < 256) s_cnt[threadIdx.x] = 0u;
  __syncthreads();
  if (b < nblk) {
    const int i = b * 1024 + threadIdx.x;
    if (i < C) atomicAdd(&s_cnt[(key[i] >> (8 * pass)) & 255u], 1u);
    __syncthreads();
    if (threadIdx.x < 256) g.rs_hist[(size_t)threadIdx.x * g.maxRs + b] = s_cnt[threadIdx.x];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const int ticket = __hip_atomic_fetch_add(&g.ctr->lru_ticket, 1, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == (int)gridDim.x - 1;
    if (ticket < 0 || ticket >= (int)gridDim.x) latch(g.ctr, ULA_ESTATE);
    if (s_last) {
      g.ctr->lru_ticket = 0;
      __threadfence();
    }
  }
  __syncthreads();
  if (!s_last) return;
  // per digit: offsets of the blocks within the digit, and the digit's total
  int tot = 0;
  if (threadIdx.x < 256) {
    uint32_t* row = g.rs_hist + (size_t)threadIdx.x * g.maxRs;
    for (int j = 0; j < nblk; ++j) {
      const uint32_t v = row[j];
      row[j] = (uint32_t)tot;
      tot += (int)v;
    }
  }
  int total;
  const int base = block_exclusive_sum<1024>(threadIdx.x < 256 ? tot : 0, scratch, total);
  if (threadIdx.x < 256) g.rs_base[threadIdx.x] = (uint32_t)base;
}

__global__ __launch_bounds__(1024) void k_rs_scatter(GroupDev g, int32_t pass) {
  constexpr int NW = 1024 / kWave;
  __shared__ int s_cnt[NW][256];
  if (block_failed(g.ctr)) return;
  if (g.ctr->n_miss == 0) return;
  const int C = g.ctr->lru_c;
  const int np = sort_passes(g.ctr->lru_kstar);
  if (pass >= np || C == 0) return;
  const int b = blockIdx.x;
  if (b >= (C + 1023) / 1024) return;   // no barrier follows for these workgroups
  const bool last = pass == np - 1;
  const uint32_t* key = g.sort_key[pass & 1];
  const uint32_t* slot = g.sort_slot[pass & 1];
  for (int i = threadIdx.x; i < NW * 256; i += blockDim.x) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  const int wave = threadIdx.x / kWave;
  const int i = b * 1024 + threadIdx.x;
  const bool valid = i < C;
  const uint32_t k = valid ? key[i] : 0u;
  const uint32_t s = valid ? slot[i] : 0u;
  const uint32_t d = (k >> (8 * pass)) & 255u;
  // lanes of this wavefront with the same digit (multisplit by eight ballots)
  unsigned long long same = __ballot(valid);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const unsigned long long bj = __ballot((d >> j) & 1u);
    same &= ((d >> j) & 1u) ? bj : ~bj;
  }
  const int rank = rank_below(same);
  if (valid && rank == 0) s_cnt[wave][d] = __popcll(same);
  __syncthreads();
  if (threadIdx.x < 256) {   // per digit: exclusive prefix over the wavefronts
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int v = s_cnt[w][threadIdx.x];
      s_cnt[w][threadIdx.x] = run;
      run += v;
    }
  }
  __syncthreads();
  if (!valid) return;
  const int pos = (int)g.rs_base[d] + (int)g.rs_hist[(size_t)d * g.maxRs + b] + s_cnt[wave][d] + rank;
  if (last) {
    g.victims[pos] = (k == 0u ? kHostBit : 0u) | s;
  } else {
    g.sort_key[(pass + 1) & 1][pos] = k;
    g.sort_slot[(pass + 1) & 1][pos] = s;
  }
}

static inline uint32_t wb_pass_step(int wbb, uint32_t t) { return wbb > 0 ? t - 1u : 0u; }

hipError_t launch_lru_select(const GroupDev& g, uint32_t t, int32_t max_pairs, int32_t wb_pairs,
                             hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  // host-link workgroups of kLruThreads lanes, four 16-byte pieces per lane per
  // round: as many bytes in flight as the mark launch's prefetch and write-back
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  constexpr int kScale = 1024 / kLruThreads;
  auto blocks_for = [&](int32_t pairs, int cap) {
    const int64_t n = ((int64_t)pairs * chunks + 4 * kLruThreads - 1) / (4 * kLruThreads);
    return (int)std::min<int64_t>(n, (int64_t)cap * kScale);
  };
  const int pf = g.H > 0 ? blocks_for(max_pairs, kPrefetchBlocks) : 0;
  const int wbb = g.H > 0 ? blocks_for(wb_pairs, kWritebackBlocks) : 0;
  // one bitmap word (32 slots) per lane: enough workgroups to spread the scan over
  // the compute units
  const int nsel = (int)std::min<int64_t>(std::max<int64_t>((g.W + kLruThreads - 1) / kLruThreads, 1), 1024);
  const FastDiv per_slot(chunks);
  // keys are at most t: the digits of bits 21-31 (and 10-20) are zero for every
  // key while t < 2^21 (2^10), and those passes would pick digit 0
  const int first = t >= (1u << 21) ? 0 : (t >= (1u << 10) ? 1 : 2);
  // the first pass also carries the host-link work (the launch ULA_TIMING_LINK times)
  if (start)
    hipExtLaunchKernelGGL(k_lru_pass, dim3(nsel + pf + wbb), dim3(kLruThreads), 0, s, start, stop, 0, g, t,
                          first, first, nsel, per_slot, pf, wbb, wb_pass_step(wbb, t));
  else
    k_lru_pass<<<nsel + pf + wbb, kLruThreads, 0, s>>>(g, t, first, first, nsel, per_slot, pf, wbb,
                                                         wb_pass_step(wbb, t));
  hipError_t e = hipGetLastError();
  for (int pass = first + 1; pass < 3 && e == hipSuccess; ++pass) {
    k_lru_pass<<<nsel, kLruThreads, 0, s>>>(g, t, pass, first, nsel, per_slot, 0, 0, 0u);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_lru_order(const GroupDev& g, uint32_t t, int32_t max_pairs, hipStream_t s) {
  constexpr int kWavesPerGroup = kSpanThreads / kWave;
  const int spans = (int)std::min<int64_t>(std::max<int64_t>((g.T + kWavesPerGroup - 1) / kWavesPerGroup, 1),
                                           4096);
  k_lru_count<<<spans, kSpanThreads, 0, s>>>(g, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_lru_emit<<<spans, kSpanThreads, 0, s>>>(g, t);
  e = hipGetLastError();
  // keys are at most t + 1: enough 8-bit passes for that (idle passes exit at once)
  int passes = 0;
  for (uint64_t x = (uint64_t)t; x; x >>= 8) ++passes;
  const int blocks = std::max(1, std::min(g.maxRs, (max_pairs + 1023) / 1024));
  for (int p = 0; p < passes && e == hipSuccess; ++p) {
    k_rs_count<<<blocks, 1024, 0, s>>>(g, p);
    e = hipGetLastError();
    if (e == hipSuccess) {
      k_rs_scatter<<<blocks, 1024, 0, s>>>(g, p);
      e = hipGetLastError();
    }
  }
  return e;
}

}  // namespace ula
