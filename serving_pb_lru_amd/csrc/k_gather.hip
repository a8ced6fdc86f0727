// Gather of the selected rows of one layer into contiguous per-set buffers.
//
// UlaCache summary (paper-daily.com): attention reads only the KV rows at the
// selected positions (introduction) and waits for the completion signal before
// reading the new locations (section 3); layers sharing one selection read the
// same entries (section 2), so this kernel runs once per layer of a group.
//
// out[j][i][:] = pool[map[sel[j][i]]][layer][:], or zeros for -1 padding. The
// work is flattened over 16-byte pieces: lane idx handles piece (idx mod C) of
// output row (idx div C), C = row_bytes / 16, so consecutive lanes write
// consecutive 16 bytes (fully coalesced, non-temporal stores) and the lanes of
// one row read one contiguous source row. Bound by HBM bandwidth.
#include "device_util.h"

namespace ula {

__global__ __launch_bounds__(256) void k_gather(GroupDev g, const int32_t* __restrict__ sel, int32_t n,
                                                int32_t layer, uint8_t* __restrict__ out,
                                                long long want_flag, FastDiv per_row) {
  if (status_of(g.ctr)) return;
  const long long f = __hip_atomic_load(&g.ctr->flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
  if (f != want_flag) {
    latch(g.ctr, ULA_ENOTRESIDENT);
    return;
  }
  const uint32_t C = (uint32_t)g.row_bytes / 16u;
  const uint32_t total = (uint32_t)n * C;
  const uint32_t stride = gridDim.x * blockDim.x;
  const uint8_t* src_base = g.pool + (size_t)layer * g.row_bytes;
  vec4u* o = reinterpret_cast<vec4u*>(out);
  constexpr int U = 4;
  int err = 0;
  for (uint32_t base = blockIdx.x * blockDim.x + threadIdx.x; base < total; base += U * stride) {
    vec4u v[U];
    int32_t la[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + u * stride;
      la[u] = idx < total ? sel[per_row.div(idx)] : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + u * stride;
      v[u] = vec4u{0u, 0u, 0u, 0u};
      if (la[u] != -1) {
        if (la[u] < 0 || la[u] >= g.N) {
          err = ULA_ERANGE;
        } else {
          const uint32_t loc = g.map[la[u]];
          if (loc & kHostBit) {
            err = ULA_ENOTRESIDENT;
          } else {
            const uint32_t c = idx - per_row.div(idx) * C;
            v[u] = reinterpret_cast<const vec4u*>(src_base + (size_t)loc * g.slot_bytes)[c];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + u * stride;
      if (idx < total) __builtin_nontemporal_store(v[u], o + idx);
    }
  }
  if (err) latch(g.ctr, err);
}

hipError_t launch_gather(const GroupDev& g, const int32_t* sel, int32_t n, int32_t layer,
                         uint8_t* out, long long want_flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const uint32_t C = (uint32_t)g.row_bytes / 16u;
  size_t total = (size_t)n * C;
  int blocks = (int)((total + 1023) / 1024);
  if (blocks > 8192) blocks = 8192;
  k_gather<<<blocks, 256, 0, s>>>(g, sel, n, layer, out, want_flag, FastDiv(C));
  return hipGetLastError();
}

}  // namespace ula
