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
// workgroup takes ROWS output rows at a time: ROWS lanes look the rows up once
// (selection entry and resolved slot in one round trip, else the mapping
// table) into LDS, then all lanes stream the rows in 16-byte pieces,
// C = row_bytes / 16 pieces per row, lane i taking piece (i mod C) of row
// (i div C): consecutive lanes write consecutive 16 bytes (fully coalesced,
// non-temporal stores) and read one contiguous source row. UNROLL pieces per
// lane are in flight; for 656-byte rows both tilings below cover all staged
// rows in one round. Bound by HBM bandwidth.
//
// Tilings (measured on MI355X with 656-byte rows): a small gather (up to 64K
// rows, a few workgroups per compute unit) is fastest with 64 rows and 11 pieces
// in flight per lane of 256; a large one (131K rows and more) with 32 rows and 3
// pieces per lane of 512, which keeps more workgroups resident.
#include <hip/hip_ext.h>

#include "device_util.h"

namespace ula {

constexpr int kSmallGatherRows = 1 << 16;   // up to this many rows: the small-gather tiling

// Rows are read with plain (cached) loads: repeated entries of one step (the
// speculative sets) and the heavy overlap between consecutive steps both hit the
// caches; non-temporal loads measured 18% slower on the speculative workload and
// only 3% faster where nothing repeats.
template <int ROWS, int UNROLL, int THREADS>
__global__ __launch_bounds__(THREADS) void k_gather(GroupDev g, const int32_t* __restrict__ sel, int32_t n,
                                                    int32_t layer, uint8_t* __restrict__ out,
                                                    long long want_flag, int32_t n_res, FastDiv per_row) {
  static_assert(ROWS < THREADS, "one lane per staged row plus the checking lane");
  __shared__ long long s_off[ROWS];   // source byte offset of each staged row, -1 = zero row
  __shared__ int s_ok;
  const uint32_t C = (uint32_t)g.row_bytes / 16u;
  const size_t layer_off = (size_t)layer * g.row_bytes;
  int err = 0;
  bool first_round = true;
  for (int row0 = blockIdx.x * ROWS; row0 < n; row0 += gridDim.x * ROWS) {
    // 1. resolve the block's rows once: the step already resolved its own
    //    selection entry by entry (res); an entry that differs from it, or lies
    //    beyond it, goes through the mapping table. In the first round thread 0
    //    checks the group's status and completion counter in the same round trip.
    //    The counter read is relaxed: ordering after the step comes from the
    //    stream (same stream, event or stream wait on the counter), whose
    //    kernel-boundary acquire already makes the moved rows visible; this
    //    check only catches a gather issued without that ordering (an acquire
    //    here would invalidate caches in every workgroup).
    if (first_round && threadIdx.x == ROWS) {
      int ok = status_of(g.ctr) == 0;
      const long long f = __hip_atomic_load(&g.ctr->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ok && f != want_flag) {
        latch(g.ctr, ULA_ENOTRESIDENT);
        ok = 0;
      }
      s_ok = ok;
    }
    if (threadIdx.x < ROWS) {
      const int r = row0 + threadIdx.x;
      long long off = -1;
      if (r < n) {
        // the selection entry and its resolved slot are loaded together (one round trip)
        const uint2 rs = r < n_res ? g.res[r] : make_uint2(kAbsent, kAbsent);
        const int32_t la = sel[r];
        if (la != -1) {
          uint32_t slot = kAbsent;
          if (r < n_res) {
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
    const int nrows = min(ROWS, n - row0);
    const uint32_t pieces = (uint32_t)nrows * C;
    vec4u* o = reinterpret_cast<vec4u*>(out) + (size_t)row0 * C;
    for (uint32_t i0 = threadIdx.x; i0 < pieces; i0 += THREADS * UNROLL) {
      vec4u v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const uint32_t i = i0 + u * THREADS;
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
      for (int u = 0; u < UNROLL; ++u) {
        const uint32_t i = i0 + u * THREADS;
        if (i < pieces) __builtin_nontemporal_store(v[u], o + i);
      }
    }
    __syncthreads();
  }
  if (err) latch(g.ctr, err);
}

template <int ROWS, int UNROLL, int THREADS>
static hipError_t launch_tiled(const GroupDev& g, const int32_t* sel, int32_t n, int32_t layer, uint8_t* out,
                               long long want_flag, int32_t n_res, hipStream_t s, hipEvent_t start,
                               hipEvent_t stop) {
  int blocks = (n + ROWS - 1) / ROWS;
  if (blocks > 32768) blocks = 32768;
  const FastDiv per_row((uint32_t)g.row_bytes / 16u);
  if (start)
    hipExtLaunchKernelGGL(k_gather<ROWS, UNROLL, THREADS>, dim3(blocks), dim3(THREADS), 0, s, start, stop, 0,
                          g, sel, n, layer, out, want_flag, n_res, per_row);
  else
    k_gather<ROWS, UNROLL, THREADS><<<blocks, THREADS, 0, s>>>(g, sel, n, layer, out, want_flag, n_res, per_row);
  return hipGetLastError();
}

hipError_t launch_gather(const GroupDev& g, const int32_t* sel, int32_t n, int32_t layer,
                         uint8_t* out, long long want_flag, int32_t n_res, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop) {
  if (n <= 0) return hipSuccess;
  if (n <= kSmallGatherRows)
    return launch_tiled<64, 11, 256>(g, sel, n, layer, out, want_flag, n_res, s, start, stop);
  return launch_tiled<32, 3, 512>(g, sel, n, layer, out, want_flag, n_res, s, start, stop);
}

}  // namespace ula
