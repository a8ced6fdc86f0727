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
// The host pool is pinned, device-mapped memory: the swap kernel reads and
// writes it directly over PCIe with 16-byte vector accesses, both directions in
// flight at once, and every lane holds both 16-byte pieces of its pair before
// writing either.
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
    const uint32_t d = g.app_dst[i];
    const vec4u v = reinterpret_cast<const vec4u*>(rows + (size_t)i * g.slot_bytes)[c];
    uint8_t* dst = (d & kHostBit) ? g.host + (size_t)(d & ~kHostBit) * g.slot_bytes
                                  : g.pool + (size_t)d * g.slot_bytes;
    reinterpret_cast<vec4u*>(dst)[c] = v;
    if (c == 0) {
      const int32_t la = g.app_la[i];
      g.map[la] = d;
      if (d & kHostBit) g.hown[d & ~kHostBit] = la;
      else g.gown[d] = la;
    }
  }
}

// Miss path: pair i swaps GPU slot victims[i] with host slot miss_h[i] for all
// layers of the group (one contiguous slot_bytes run on each side).
__global__ __launch_bounds__(256) void k_swap(GroupDev g, FastDiv per_slot) {
  if (status_of(g.ctr)) return;
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t total = (uint32_t)g.ctr->n_miss * chunks;
  const uint32_t stride = gridDim.x * blockDim.x;
  constexpr int U = 4;
  for (uint32_t base = blockIdx.x * blockDim.x + threadIdx.x; base < total; base += U * stride) {
    vec4u hv[U], gv[U];
    vec4u* gp[U];
    vec4u* hp[U];
    bool ev[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + u * stride;
      ev[u] = false;
      gp[u] = nullptr;
      if (idx < total) {
        const uint32_t i = per_slot.div(idx);
        const uint32_t c = idx - i * chunks;
        const uint32_t v = g.victims[i];
        const uint32_t h = g.miss_h[i];
        ev[u] = g.gown[v] != -1;
        gp[u] = reinterpret_cast<vec4u*>(g.pool + (size_t)v * g.slot_bytes) + c;
        hp[u] = reinterpret_cast<vec4u*>(g.host + (size_t)h * g.slot_bytes) + c;
        hv[u] = *hp[u];
        if (ev[u]) gv[u] = *gp[u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (gp[u]) {
        *gp[u] = hv[u];
        if (ev[u]) *hp[u] = gv[u];
      }
    }
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
    const uint32_t v = g.victims[i];
    const int32_t la = g.miss_la[i];
    const uint32_t h = g.miss_h[i];
    const int32_t old = g.gown[v];
    g.map[la] = v;
    g.gown[v] = la;
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
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (s_freed) atomicAdd(&g.ctr->hfree, s_freed);
    __threadfence();
    const int ticket = atomicAdd(&g.ctr->done, 1);
    if (ticket == (int)gridDim.x - 1) {
      g.ctr->done = 0;
      __threadfence_system();
      __hip_atomic_store(&g.ctr->flag, t, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
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

hipError_t launch_swap(const GroupDev& g, int32_t max_pairs, hipStream_t s) {
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  size_t total = (size_t)max_pairs * chunks;
  int blocks = (int)((total + 1023) / 1024);
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  k_swap<<<blocks, 256, 0, s>>>(g, FastDiv(chunks));
  return hipGetLastError();
}

hipError_t launch_commit(const GroupDev& g, long long t, hipStream_t s) {
  k_commit<<<256, 256, 0, s>>>(g, t);
  return hipGetLastError();
}

}  // namespace ula
