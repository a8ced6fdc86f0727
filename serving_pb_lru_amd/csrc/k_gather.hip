// Gather of the selected rows of one layer into contiguous per-set buffers.
//
// UlaCache summary (paper-daily.com): attention reads only the KV rows at the
// selected positions (introduction) and waits for the completion signal before
// reading the new locations (section 3); layers sharing one selection read the
// same entries (section 2), so this kernel runs once per layer of a group.
//
// out[j][i][:] = pool[map[sel[j][i]]][layer][:], or zeros for -1 padding. A
// workgroup takes 32 output rows at a time: 32 lanes look the rows up once
// (selection entry, then mapping table) into LDS, then all 256 lanes stream
// the rows in 16-byte pieces, C = row_bytes / 16 pieces per row, lane i taking
// piece (i mod C) of row (i div C): consecutive lanes write consecutive 16
// bytes (fully coalesced, non-temporal stores) and read one contiguous source
// row. Six pieces per lane are in flight (one round for 656-byte rows). Bound
// by HBM bandwidth.
#include "device_util.h"

namespace ula {

constexpr int kGatherRows = 32;   // output rows staged per workgroup iteration
constexpr int kGatherUnroll = 6;  // 16-byte pieces in flight per lane

__global__ __launch_bounds__(256) void k_gather(GroupDev g, const int32_t* __restrict__ sel, int32_t n,
                                                int32_t layer, uint8_t* __restrict__ out,
                                                long long want_flag, FastDiv per_row) {
  __shared__ long long s_off[kGatherRows];   // source byte offset of each staged row, -1 = zero row
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    int ok = status_of(g.ctr) == 0;
    if (ok) {
      // A relaxed read: ordering after the step comes from the stream (same
      // stream, event or stream wait on the counter), whose kernel-boundary
      // acquire already makes the moved rows visible; this check only catches
      // a gather issued without that ordering. An acquire here would
      // invalidate caches in every workgroup.
      const long long f = __hip_atomic_load(&g.ctr->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (f != want_flag) {
        latch(g.ctr, ULA_ENOTRESIDENT);
        ok = 0;
      }
    }
    s_ok = ok;
  }
  __syncthreads();
  if (!s_ok) return;
  const uint32_t C = (uint32_t)g.row_bytes / 16u;
  const size_t layer_off = (size_t)layer * g.row_bytes;
  int err = 0;
  for (int row0 = blockIdx.x * kGatherRows; row0 < n; row0 += gridDim.x * kGatherRows) {
    // 1. look up the block's rows once: selection entry -> mapping table -> offset
    if (threadIdx.x < kGatherRows) {
      const int r = row0 + threadIdx.x;
      long long off = -1;
      if (r < n) {
        const int32_t la = sel[r];
        if (la != -1) {
          if (la < 0 || la >= g.N) {
            err = ULA_ERANGE;
          } else {
            const uint32_t loc = g.map[la];
            if (loc & kHostBit) err = ULA_ENOTRESIDENT;
            else off = (long long)((size_t)loc * g.slot_bytes + layer_off);
          }
        }
      }
      s_off[threadIdx.x] = off;
    }
    __syncthreads();
    // 2. stream the staged rows: piece i of the block is piece (i mod C) of row (i div C)
    const int nrows = min(kGatherRows, n - row0);
    const uint32_t pieces = (uint32_t)nrows * C;
    vec4u* o = reinterpret_cast<vec4u*>(out) + (size_t)row0 * C;
    for (uint32_t i0 = threadIdx.x; i0 < pieces; i0 += blockDim.x * kGatherUnroll) {
      vec4u v[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const uint32_t i = i0 + u * blockDim.x;
        v[u] = vec4u{0u, 0u, 0u, 0u};
        if (i < pieces) {
          const uint32_t r = per_row.div(i);
          const long long off = s_off[r];
          if (off >= 0) v[u] = *reinterpret_cast<const vec4u*>(g.pool + off + (size_t)(i - r * C) * 16);
        }
      }
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const uint32_t i = i0 + u * blockDim.x;
        if (i < pieces) __builtin_nontemporal_store(v[u], o + i);
      }
    }
    __syncthreads();
  }
  if (err) latch(g.ctr, err);
}

hipError_t launch_gather(const GroupDev& g, const int32_t* sel, int32_t n, int32_t layer,
                         uint8_t* out, long long want_flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int blocks = (n + kGatherRows - 1) / kGatherRows;
  if (blocks > 4096) blocks = 4096;
  k_gather<<<blocks, 256, 0, s>>>(g, sel, n, layer, out, want_flag, FastDiv((uint32_t)g.row_bytes / 16u));
  return hipGetLastError();
}

}  // namespace ula
