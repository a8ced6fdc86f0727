// Data movement and commit: append placement, the HBM part of the miss-path
// swap, and the commit that updates the mapping table and signals completion.
//
// Ordering (UlaCache summary, paper-daily.com, section 3): rows land before the
// mapping table names their new slots, and the completion counter is raised
// last, so a reader that waits for the counter only sees finished moves. Pools
// (section 2): each entry is held by exactly one of the GPU and host pools. Here the i-th miss takes the i-th victim slot, the
// missed rows come in from the miss's host slot and the victim's rows go out
// to that same host slot (a swap), so host occupancy is unchanged and no entry
// is ever held twice; a victim taken from the free bucket frees the host slot.
//
// The miss path runs in three parts: the missed rows are read into HBM early
// (prefetch workgroups of the mark launch), the swap into the victim slots is
// HBM to HBM (here), and the evicted rows, staged in HBM by the swap, go to the
// host in the next step's mark launch, beside that step's reads.
#include <algorithm>

#include "miss_path.h"

namespace ula {

// Append: destinations were chosen by the plan/extract pair (app_dst). Copy
// rows in 16-byte pieces and publish map/owner entries.
__global__ __launch_bounds__(256) void k_place(GroupDev g, int32_t n, const uint8_t* __restrict__ rows,
                                               FastDiv per_slot) {
  if (status_of(g.ctr)) return;
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t total = (uint32_t)n * chunks;
  for (uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += gridDim.x * blockDim.x) {
    const uint32_t i = per_slot.div(idx);
    const uint32_t c = idx - i * chunks;
    const vec4u v = reinterpret_cast<const vec4u*>(rows + (size_t)i * g.slot_bytes)[c];
    place_piece(g, g.app_dst[i], c, c == 0 ? g.app_la[i] : 0, v);
  }
}

// Append under ULA_PLACE_RING: destinations from the plan/extract pair (app_dst:
// the GPU slots taken, then the host slots), the counts from the plan.
__global__ __launch_bounds__(256) void k_place_ring(GroupDev g, int32_t n, const uint8_t* __restrict__ rows,
                                                    FastDiv per_slot) {
  __shared__ int s_status, s_q[2];
  if (threadIdx.x == 0) s_status = status_of(g.ctr);
  else if (threadIdx.x == kWave) s_q[0] = g.ctr->app_q;
  else if (threadIdx.x == 2 * kWave) s_q[1] = g.ctr->app_qfree;
  __syncthreads();
  if (s_status) return;
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t total = (uint32_t)n * chunks;
  for (uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += gridDim.x * blockDim.x) {
    const uint32_t i = per_slot.div(idx);
    const uint32_t c = idx - i * chunks;
    const vec4u v = reinterpret_cast<const vec4u*>(rows + (size_t)i * g.slot_bytes)[c];
    place_piece_ring(g, g.app_dst, s_q[0], s_q[1], i, c, c == 0 ? g.app_la[i] : 0, v);
  }
}

// Miss path, HBM part, fused with the commit. Pair i moves the missed rows,
// already prefetched into miss_rows[i], into victim slot victims[i]; a victim
// that holds an entry first copies its rows to the staging buffer, from which
// the next step's mark launch (or a stand-alone write-back before the host
// reads state) writes them to the host slot the miss vacated. Each pair is also
// committed (commit_pair): beside its first piece when one round of the data
// loop covers every piece, else one lane per pair after the loop. The
// completion counter is raised by k_publish, launched right after on the same
// stream: the kernel boundary makes every workgroup's writes visible first. (A
// release fence and a ticket in every workgroup, so that the last one could
// raise it, wrote each compute die's L2 back once per workgroup and cost about a
// third of this kernel.)
// Commit of pair i: mapping table, owners, the step's resolved selection, and
// the staging record of the host slot; a victim that was free releases its host
// slot instead (counted in `freed`).
__device__ __forceinline__ void commit_pair(const GroupDev& g, uint32_t t, int i, int& freed) {
  const uint32_t v = g.victims[i] & ~kHostBit;
  const int32_t la = g.miss_la[i];
  const uint32_t h = g.miss_h[i];
  const int32_t old = g.gown[v];
  g.map[la] = v;
  g.gown[v] = la;
  if (g.lru_ts) g.lru_ts[v] = (int32_t)t;   // exact LRU: loaded this step
  g.res[g.miss_e[i]].y = v;      // the step's selection now resolves to the loaded slot
  if (old != -1) {
    g.map[old] = kHostBit | h;
    g.hown[h] = old;
    g.wb_h[i] = h;
    g.hs_stage[h] = ((unsigned long long)t << 32) | (uint32_t)i;
  } else {
    g.hown[h] = -1;
    g.wb_h[i] = kAbsent;
    atomicOr(&g.hbm[h >> 5], 1u << (h & 31));
    atomicAdd(&g.htcnt[h >> kTileShift], 1u);
    atomicMin(&g.ctr->hfree_lo, (int32_t)(h >> kTileShift));
    ++freed;
  }
}

__global__ __launch_bounds__(512) void k_swap_commit(GroupDev g, uint32_t t, FastDiv per_slot) {
  __shared__ int s_freed, s_status, s_m;
  // the error status and the pair count in one round trip
  if (threadIdx.x == 0) {
    s_status = status_of(g.ctr);
    s_freed = 0;
  } else if (threadIdx.x == kWave) {
    s_m = g.ctr->n_miss;
  }
  __syncthreads();
  if (s_status) return;
  const int m = s_m;
  uint8_t* stage = g.evict_rows;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    g.ctr->wb_n = m;
    g.ctr->wb_step = t;
    g.ctr->mark_role = 0;   // the mark launch has ended: every workgroup took its role
  }
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t total = (uint32_t)m * chunks;
  const uint32_t stride = gridDim.x * blockDim.x;
  int freed = 0;
  constexpr int U = 4;
  const bool one_round = total <= U * stride;
  for (uint32_t base = blockIdx.x * blockDim.x + threadIdx.x; base < total; base += U * stride) {
    vec4u mv[U], gv[U];
    vec4u* gp[U];
    vec4u* sp[U];
    bool ev[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + u * stride;
      gp[u] = nullptr;
      ev[u] = false;
      if (idx < total) {
        const uint32_t i = per_slot.div(idx);
        const uint32_t c = idx - i * chunks;
        const uint32_t vv = g.victims[i];
        const uint32_t v = vv & ~kHostBit;
        ev[u] = (vv & kHostBit) == 0;          // the victim slot holds an entry to evict
        gp[u] = reinterpret_cast<vec4u*>(g.pool + (size_t)v * g.slot_bytes) + c;
        sp[u] = reinterpret_cast<vec4u*>(stage + (size_t)i * g.slot_bytes) + c;
        if (ev[u]) gv[u] = *gp[u];
        mv[u] = reinterpret_cast<const vec4u*>(g.miss_rows + (size_t)i * g.slot_bytes)[c];
        // one data round covers every piece: commit beside the first piece, so
        // the commit's dependent loads overlap the row loads
        if (one_round && c == 0) commit_pair(g, t, (int)i, freed);
      }
    }
    // The staged copy is read again only by the next step's write-back:
    // non-temporal stores keep it from displacing what the step's gathers read
    // next (on the eviction-heavy workload the following gather took 174 us
    // after cached stores and 146 us after these). The rows moved into the
    // victim slots are what those gathers read, so they stay cached.
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (gp[u]) {
        if (ev[u]) __builtin_nontemporal_store(gv[u], sp[u]);
        *gp[u] = mv[u];
      }
    }
  }
  // More rounds: commit one lane per pair after the data loop (interleaved, the
  // commit's chain of dependent loads would stall a wavefront in every round).
  if (!one_round)
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < m; i += gridDim.x * blockDim.x)
      commit_pair(g, t, i, freed);
  if (g.lru_ts) {
    // exact LRU: the step's hits take its timestamp now that it has succeeded
    const int nh = g.ctr->n_hits;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nh; i += gridDim.x * blockDim.x)
      g.lru_ts[g.hit_slots[i]] = (int32_t)t;
  }
  if (freed) atomicAdd(&s_freed, freed);
  __syncthreads();
  if (threadIdx.x == 0 && s_freed) atomicAdd(&g.ctr->hfree, s_freed);
}

// The step's signal (section 3: readers wait for it): completion counter = t,
// unless an error was latched, in which case the step did not take effect. The
// store needs no release of its own: the swap's writes were made visible at
// the end of its kernel, before this one started, and this kernel's end makes
// the counter visible to other streams and the host.
// A step that failed on the device leaves the counter at the last completed
// step but sets kFlagFailed in it, so that a stream waiting for the counter to
// reach this step (hipStreamWaitValue64, "greater or equal") is released
// instead of waiting forever; a gather it then runs finds the latched status
// and refuses.
__global__ __launch_bounds__(64) void k_publish(GroupDev g, uint32_t t) {
  if (threadIdx.x != 0) return;
  if (!status_of(g.ctr))
    __hip_atomic_store(&g.ctr->flag, (long long)t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    __hip_atomic_fetch_or(&g.ctr->flag, kFlagFailed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stand-alone write-back of whatever rows the last swap staged, for when the
// host is about to read state. It does not test the error status: an error
// latched by a later step (whose mark launch then never wrote these rows out)
// must not stop the write-back of an earlier completed one. Rewriting rows a
// mark launch already wrote out is harmless: nothing else writes those host
// slots meanwhile.
__global__ __launch_bounds__(256) void k_writeback(GroupDev g, FastDiv per_slot) {
  const uint32_t t = g.ctr->wb_step;
  const int n = g.ctr->wb_n;
  if (t != 0) writeback_rows(g, t, n, t, per_slot, blockIdx.x, gridDim.x);
}

// Release of finished entries (app_la[0..n), validated on the host): a GPU slot
// leaves whichever bucket holds it and joins the free set, a host slot joins the
// free host set (its staging record cleared, so no later miss reads a staged
// copy of the released row); the address becomes absent. Bucket words and span
// counts are shared between threads, hence atomics. Any staged write-back has
// been written out before this kernel runs.
__global__ __launch_bounds__(256) void k_release(GroupDev g, int32_t n) {
  if (status_of(g.ctr)) return;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int32_t la = g.app_la[i];
    const uint32_t loc = g.map[la];
    if (loc == kAbsent) {          // the host checked this: an inconsistent state
      latch(g.ctr, ULA_ESTATE);
      continue;
    }
    g.map[la] = kAbsent;
    if (loc & kHostBit) {
      const uint32_t h = loc & ~kHostBit;
      g.hown[h] = -1;
      g.hs_stage[h] = ~0ull;
      atomicOr(&g.hbm[h >> 5], 1u << (h & 31));
      atomicAdd(&g.htcnt[h >> kTileShift], 1u);
      atomicAdd(&g.ctr->hfree, 1);
      atomicMin(&g.ctr->hfree_lo, (int32_t)(h >> kTileShift));
      continue;
    }
    const uint32_t s = loc;
    const uint32_t bit = 1u << (s & 31);
    const int w = (int)(s >> 5), tile = (int)(s >> kTileShift);
    for (int id = kCold; id < g.NB; ++id) {     // the bucket holding the slot, if any
      if (g.bm[(size_t)id * g.W + w] & bit) {
        atomicAnd(&g.bm[(size_t)id * g.W + w], ~bit);
        atomicSub(&g.tcnt[(size_t)id * g.T + tile], 1u);
        atomicSub(&g.ctr->bcnt[id], 1);
        break;
      }
    }
    atomicOr(&g.bm[(size_t)kFree * g.W + w], bit);
    atomicAdd(&g.tcnt[(size_t)kFree * g.T + tile], 1u);
    atomicAdd(&g.ctr->bcnt[kFree], 1);
    atomicMin(&g.ctr->free_lo, tile);
    g.gown[s] = -1;
    if (g.lru_ts) g.lru_ts[s] = 0;   // exact LRU: a slot appended later counts as never stamped
  }
}

hipError_t launch_release(const GroupDev& g, int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  k_release<<<blocks, 256, 0, s>>>(g, n);
  return hipGetLastError();
}

hipError_t launch_place(const GroupDev& g, int32_t n, const uint8_t* rows, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  size_t total = (size_t)n * chunks;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  k_place<<<blocks, 256, 0, s>>>(g, n, rows, FastDiv(chunks));
  return hipGetLastError();
}

hipError_t launch_place_ring(const GroupDev& g, int32_t n, const uint8_t* rows, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  size_t total = (size_t)n * chunks;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  k_place_ring<<<blocks, 256, 0, s>>>(g, n, rows, FastDiv(chunks));
  return hipGetLastError();
}

static int grid_for_pairs(int32_t max_pairs, uint32_t chunks, int threads, int cap) {
  size_t total = (size_t)max_pairs * chunks;
  size_t per_block = (size_t)threads * 4;
  int blocks = (int)std::min<size_t>((total + per_block - 1) / per_block, (size_t)cap);
  return blocks < 1 ? 1 : blocks;
}

hipError_t launch_swap_commit(const GroupDev& g, uint32_t t, int32_t max_pairs, hipStream_t s) {
  // At most 256 workgroups (one per compute unit): one round of the data loop
  // then covers about 1000 three-layer pairs, so those steps commit beside it.
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  k_swap_commit<<<grid_for_pairs(max_pairs, chunks, 512, 256), 512, 0, s>>>(g, t, FastDiv(chunks));
  k_publish<<<1, 64, 0, s>>>(g, t);
  return hipGetLastError();
}

hipError_t launch_writeback(const GroupDev& g, int32_t max_pairs, hipStream_t s) {
  // 64 workgroups keep about 1 MB of stores in flight, enough to saturate the link
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  k_writeback<<<grid_for_pairs(max_pairs, chunks, 256, 64), 256, 0, s>>>(g, FastDiv(chunks));
  return hipGetLastError();
}

}  // namespace ula
