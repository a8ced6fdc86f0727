// Data movement and commit: append placement, the miss-path swap over the host
// link, and the commit that updates the mapping table and signals completion.
//
// UlaCache summary (paper-daily.com), section 3: move the data first, then
// update the mapping and signal completion; readers wait for the signal, so
// they never see half-moved data. Section 2: an entry lives in the GPU pool or
// the host pool, never both. Here the i-th miss takes the i-th victim slot, the
// missed rows come in from the miss's host slot and the victim's rows go out
// to that same host slot (a swap), so host occupancy is unchanged and no entry
// is ever held twice; a victim taken from the free bucket frees the host slot.
//
// The host pool is pinned, device-mapped memory that the kernels read and
// write directly over PCIe with 16-byte vector accesses. PCIe keeps read
// requests behind earlier posted writes in the same direction, so a swap that
// mixes both stalls its reads on its own write-back; the miss path therefore
// splits: reads into the pool first (critical path), then the write-back of
// the evicted rows from an HBM staging copy on a side stream.
#include "device_util.h"

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
    place_piece(g, i, c, c == 0 ? g.app_la[i] : 0, rows);
  }
}

// Miss path, critical part: pair i brings the missed rows of host slot
// miss_h[i] into GPU slot victims[i] (all layers: one contiguous slot_bytes run
// on each side). The victim's own rows are first copied to an HBM staging row
// so that the slot can be overwritten at once; only reads cross the host link
// here, so no read request queues behind write traffic.
__global__ __launch_bounds__(256) void k_swap_in(GroupDev g, FastDiv per_slot) {
  if (status_of(g.ctr)) return;
  const int m = g.ctr->n_miss;
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t total = (uint32_t)m * chunks;
  const uint32_t stride = gridDim.x * blockDim.x;
  if (blockIdx.x == 0 && threadIdx.x == 0) g.ctr->wb_n = m;
  constexpr int U = 4;
  for (uint32_t base = blockIdx.x * blockDim.x + threadIdx.x; base < total; base += U * stride) {
    vec4u hv[U], gv[U];
    vec4u* gp[U];
    const vec4u* hp[U];
    vec4u* sp[U];
    bool ev[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + u * stride;
      ev[u] = false;
      gp[u] = nullptr;
      if (idx < total) {
        const uint32_t i = per_slot.div(idx);
        const uint32_t c = idx - i * chunks;
        const uint32_t vv = g.victims[i];
        const uint32_t h = g.miss_h[i];
        const uint32_t v = vv & ~kHostBit;
        ev[u] = (vv & kHostBit) == 0;          // the victim slot holds a row to evict
        gp[u] = reinterpret_cast<vec4u*>(g.pool + (size_t)v * g.slot_bytes) + c;
        hp[u] = reinterpret_cast<const vec4u*>(g.host + (size_t)h * g.slot_bytes) + c;
        sp[u] = reinterpret_cast<vec4u*>(g.evict_rows + (size_t)i * g.slot_bytes) + c;
        if (ev[u]) gv[u] = *gp[u];
        hv[u] = *hp[u];
        if (c == 0) g.wb_h[i] = ev[u] ? h : kAbsent;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (gp[u]) {
        if (ev[u]) *sp[u] = gv[u];
        *gp[u] = hv[u];
      }
    }
  }
}

// Miss path, deferred part (side stream): the staged victim rows go to the host
// slots their misses vacated. It is launched when the group's next step starts
// and overlaps that step's lookup and selection; the next k_swap_in waits for
// it, so a later read of one of these host slots always sees the written row.
// It depends only on wb_n / wb_h / evict_rows, which no kernel rewrites before
// that wait.
__global__ __launch_bounds__(256) void k_writeback(GroupDev g, FastDiv per_slot) {
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t total = (uint32_t)g.ctr->wb_n * chunks;
  const uint32_t stride = gridDim.x * blockDim.x;
  constexpr int U = 4;
  for (uint32_t base = blockIdx.x * blockDim.x + threadIdx.x; base < total; base += U * stride) {
    vec4u v[U];
    vec4u* hp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + u * stride;
      hp[u] = nullptr;
      if (idx < total) {
        const uint32_t i = per_slot.div(idx);
        const uint32_t c = idx - i * chunks;
        const uint32_t h = g.wb_h[i];
        if (h != kAbsent) {
          hp[u] = reinterpret_cast<vec4u*>(g.host + (size_t)h * g.slot_bytes) + c;
          v[u] = reinterpret_cast<const vec4u*>(g.evict_rows + (size_t)i * g.slot_bytes)[c];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (hp[u]) *hp[u] = v[u];
  }
}

// Commit after the data has moved: mapping table and owners; a victim that was
// free releases its host slot. Then the last workgroup to finish raises the
// completion counter to t with a system-scope release.
__global__ __launch_bounds__(256) void k_commit(GroupDev g, long long t) {
  __shared__ int s_freed;
  if (block_failed(g.ctr)) return;
  if (threadIdx.x == 0) s_freed = 0;
  __syncthreads();
  const int m = g.ctr->n_miss;
  int freed = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < m; i += gridDim.x * blockDim.x) {
    const uint32_t v = g.victims[i] & ~kHostBit;
    const int32_t la = g.miss_la[i];
    const uint32_t h = g.miss_h[i];
    const int32_t old = g.gown[v];
    g.map[la] = v;
    g.gown[v] = la;
    g.res[g.miss_e[i]].y = v;      // the step's selection now resolves to the loaded slot
    if (old != -1) {
      g.map[old] = kHostBit | h;
      g.hown[h] = old;
    } else {
      g.hown[h] = -1;
      atomicOr(&g.hbm[h >> 5], 1u << (h & 31));
      atomicAdd(&g.htcnt[h >> kTileShift], 1u);
      ++freed;
    }
  }
  if (freed) atomicAdd(&s_freed, freed);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (s_freed) atomicAdd(&g.ctr->hfree, s_freed);
    // The barrier ordered the workgroup's writes before this thread; one
    // release per workgroup publishes them (a fence per thread would write the
    // cache back once per thread). The ticket is acquire-release, so the last
    // workgroup's release of the counter covers every workgroup's writes.
    __threadfence();
    const int ticket = __hip_atomic_fetch_add(&g.ctr->done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (ticket == (int)gridDim.x - 1) {
      g.ctr->done = 0;
      __hip_atomic_store(&g.ctr->flag, t, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
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

static int grid_for_pairs(int32_t max_pairs, uint32_t chunks) {
  size_t total = (size_t)max_pairs * chunks;
  int blocks = (int)((total + 1023) / 1024);
  if (blocks > 2048) blocks = 2048;
  return blocks < 1 ? 1 : blocks;
}

hipError_t launch_swap_in(const GroupDev& g, int32_t max_pairs, hipStream_t s) {
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  k_swap_in<<<grid_for_pairs(max_pairs, chunks), 256, 0, s>>>(g, FastDiv(chunks));
  return hipGetLastError();
}

hipError_t launch_writeback(const GroupDev& g, int32_t max_pairs, hipStream_t s) {
  // 64 workgroups keep about 1 MB of stores in flight, enough to saturate the
  // link; more would only hold compute units the concurrent kernels need.
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  int blocks = grid_for_pairs(max_pairs, chunks);
  if (blocks > 64) blocks = 64;
  k_writeback<<<blocks, 256, 0, s>>>(g, FastDiv(chunks));
  return hipGetLastError();
}

hipError_t launch_commit(const GroupDev& g, long long t, int32_t max_pairs, hipStream_t s) {
  // few workgroups: each one takes a ticket on one counter to find the last
  int blocks = (max_pairs + 4095) / 4096;
  if (blocks > 32) blocks = 32;
  if (blocks < 1) blocks = 1;
  k_commit<<<blocks, 256, 0, s>>>(g, t);
  return hipGetLastError();
}

}  // namespace ula
