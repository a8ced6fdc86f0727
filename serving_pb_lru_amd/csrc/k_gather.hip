// Gather of the selected rows of one layer into contiguous per-set buffers.
//
// UlaCache summary (paper-daily.com): attention reads only the KV rows at the
// selected positions (introduction) and waits for the completion signal before
// reading the new locations (section 3); layers sharing one selection read the
// same entries (section 2), so this kernel runs once per layer of a group.
//
// out[j][i][:] = pool[map[sel[j][i]]][layer][:], or zeros for -1 padding. The
// step already resolved its selection to slots entry by entry (the lookup is
// done once per group); a gather of that selection reads those slots in order
// and only entries that differ fall back to the mapping table. A
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

// Rows are read with plain (cached) loads: repeated entries of one step (the
// speculative sets) and the heavy overlap between consecutive steps both hit the
// caches; non-temporal loads measured 18% slower on the speculative workload and
// only 3% faster where nothing repeats.
__global__ __launch_bounds__(256) void k_gather(GroupDev g, const int32_t* __restrict__ sel, int32_t n,
                                                int32_t layer, uint8_t* __restrict__ out,
                                                long long want_flag, int32_t n_res, FastDiv per_row) {
  __shared__ long long s_off[kGatherRows];   // source byte offset of each staged row, -1 = zero row
  __shared__ int s_ok;
  const uint32_t C = (uint32_t)g.row_bytes / 16u;
  const size_t layer_off = (size_t)layer * g.row_bytes;
  int err = 0;
  bool first_round = true;
  for (int row0 = blockIdx.x * kGatherRows; row0 < n; row0 += gridDim.x * kGatherRows) {
    // 1. resolve the block's rows once: the step already resolved its own
    //    selection entry by entry (res); an entry that differs from it, or lies
    //    beyond it, goes through the mapping table. In the first round thread 0
    //    checks the group's status and completion counter in the same round trip.
    //    The counter read is relaxed: ordering after the step comes from the
    //    stream (same stream, event or stream wait on the counter), whose
    //    kernel-boundary acquire already makes the moved rows visible; this
    //    check only catches a gather issued without that ordering (an acquire
    //    here would invalidate caches in every workgroup).
    if (first_round && threadIdx.x == kGatherRows) {
      int ok = status_of(g.ctr) == 0;
      const long long f = __hip_atomic_load(&g.ctr->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ok && f != want_flag) {
        latch(g.ctr, ULA_ENOTRESIDENT);
        ok = 0;
      }
      s_ok = ok;
    }
    if (threadIdx.x < kGatherRows) {
      const int r = row0 + threadIdx.x;
      long long off = -1;
      if (r < n) {
        const int32_t la = sel[r];
        if (la != -1) {
          uint32_t slot = kAbsent;
          if (r < n_res) {
            const uint2 rs = g.res[r];
            if (rs.x == (uint32_t)la) {
              slot = rs.y;
              if ((slot & kHostBit) && slot != kAbsent && (int32_t)(slot & ~kHostBit) < n_res) {
                const uint2 first = g.res[slot & ~kHostBit];      // a repeated miss
                slot = first.x == (uint32_t)la ? first.y : kAbsent;
              }
            }
          }
          if (slot & kHostBit) {
            if (la < 0 || la >= g.N) {
              err = ULA_ERANGE;
            } else {
              const uint32_t loc = g.map[la];
              if (loc & kHostBit) err = ULA_ENOTRESIDENT;
              else slot = loc;
            }
          }
          if (!(slot & kHostBit)) off = (long long)((size_t)slot * g.slot_bytes + layer_off);
        }
      }
      s_off[threadIdx.x] = off;
    }
    __syncthreads();
    if (first_round) {
      if (!s_ok) return;   // block-uniform
      first_round = false;
    }
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
          if (off >= 0) {
            const vec4u* p = reinterpret_cast<const vec4u*>(g.pool + off + (size_t)(i - r * C) * 16);
            v[u] = *p;
          }
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
                         uint8_t* out, long long want_flag, int32_t n_res, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int blocks = (n + kGatherRows - 1) / kGatherRows;
  if (blocks > 32768) blocks = 32768;
  k_gather<<<blocks, 256, 0, s>>>(g, sel, n, layer, out, want_flag, n_res,
                                  FastDiv((uint32_t)g.row_bytes / 16u));
  return hipGetLastError();
}

}  // namespace ula
