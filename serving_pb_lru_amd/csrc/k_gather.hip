// Gather of the selected rows of one or more layers into contiguous per-set
// buffers.
//
// UlaCache summary (paper-daily.com): attention reads only the KV rows at the
// selected positions (introduction) and waits for the completion signal before
// reading the new locations (section 3); layers sharing one selection read the
// same entries (section 2), so a group's layers are gathered one launch per
// layer, or several in one launch: the later layers of a group are fetched
// together while the first one is in use (section 2).
//
// out[l][j][i][:] = pool[map[sel[j][i]]][layer0 + l][:] for the nl layers of
// one launch (one per-layer buffer each, layer_stride apart), or zeros for -1
// padding. A slot keeps its layers side by side, so the nl rows of one entry
// are one contiguous source run. The step already resolved its selection to
// slots entry by entry (the lookup is done once per group); a gather of that
// selection reads those slots in order and only entries that differ fall back
// to the mapping table. A workgroup takes ROWS output rows at a time: ROWS
// lanes look the rows up once (selection entry and resolved slot in one round
// trip, else the mapping table) into LDS, then all lanes stream the rows in
// 16-byte pieces, C = row_bytes / 16 pieces per row, lane i taking piece
// (i mod C) of row (i div C), layer by layer: consecutive lanes write
// consecutive 16 bytes (fully coalesced, non-temporal stores) and read one
// contiguous source row.
// UNROLL pieces per lane are in flight; for 656-byte rows both tilings below
// cover all staged rows of one layer in one round. Bound by HBM bandwidth.
//
// Tilings (measured on MI355X with 656-byte rows): a small gather is fastest
// when each workgroup's rows take one round of 11 pieces per lane of 256: 64
// rows for one layer (up to 64K rows), 32 rows for two layers and 16 for three
// or more (up to 128K row-layers; the two-layer launch of 32K rows 16.5 against
// 18.5 us with 64 rows, the three-layer one 24.8 against 25.5 us with the large
// tiling); larger launches take 32 rows and 3 pieces per lane of 512, which
// keeps more workgroups resident.
#include <hip/hip_ext.h>

#include "device_util.h"

namespace ula {

constexpr int kSmallGatherRows = 1 << 16;   // up to this many rows (one layer): the small-gather tiling

// Streams the staged rows of one block, layer by layer: piece i is piece
// (i mod C) of staged row q = i div C, which is row (q mod nrows) of layer
// (q div nrows); layer l's output rows start layer_stride pieces after layer
// l - 1's. s_off[r]: source offset of row r's first layer (-1: zero row).
// MULTI = false is the one-layer case, without the layer arithmetic.
// NT: rows are read with non-temporal loads. A one-layer gather of a step whose
// selection repeats no entry reads every row once, so it does (measured: 17%
// faster on the eviction-heavy workload, whose rows come cold after the swap,
// and the next step's lookups find more of their tables in the caches). Other
// gathers use plain loads: repeated entries (the speculative sets) and the
// neighbouring layers of one slot (a 128-byte line spans two of them) hit the
// caches, and non-temporal loads there measured 18% and 14% slower. Output
// pieces are written with non-temporal stores: plain stores measured 5-12%
// slower per launch.
template <int ROWS, int UNROLL, int THREADS, bool MULTI, bool NT>
__device__ __forceinline__ void stream_rows(const GroupDev& g, const long long* s_off, int nrows, int nl,
                                            size_t layer_stride, vec4u* o, uint32_t C, FastDiv per_row) {
  const uint32_t per_layer = (uint32_t)nrows * C;
  const uint32_t pieces = MULTI ? per_layer * (uint32_t)nl : per_layer;
  for (uint32_t i0 = threadIdx.x; i0 < pieces; i0 += THREADS * UNROLL) {
    vec4u v[UNROLL];
    vec4u* dst[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t i = i0 + u * THREADS;
      v[u] = vec4u{0u, 0u, 0u, 0u};
      dst[u] = nullptr;
      if (i < pieces) {
        const uint32_t q = per_row.div(i);
        uint32_t l = 0, r = q;
        if (MULTI) {
          if (nrows == ROWS) {   // block-uniform: every block but the last
            l = q / ROWS;
            r = q % ROWS;
          } else {
            l = q / (uint32_t)nrows;
            r = q - l * (uint32_t)nrows;
          }
        }
        const long long off = s_off[r];
        if (off >= 0) {
          const vec4u* p = reinterpret_cast<const vec4u*>(g.pool + off + (size_t)l * g.row_bytes +
                                                          (size_t)(i - q * C) * 16);
          if constexpr (NT) v[u] = __builtin_nontemporal_load(p);
          else v[u] = *p;
        }
        dst[u] = MULTI ? o + (size_t)l * layer_stride + (i - l * per_layer) : o + i;
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (dst[u]) __builtin_nontemporal_store(v[u], dst[u]);
  }
}

template <int ROWS, int UNROLL, int THREADS>
__global__ __launch_bounds__(THREADS) void k_gather(GroupDev g, const int32_t* __restrict__ sel, int32_t n,
                                                    int32_t layer, int32_t nl, size_t layer_stride,
                                                    uint8_t* __restrict__ out, long long want_flag,
                                                    int32_t n_res, FastDiv per_row) {
  static_assert(ROWS < THREADS, "one lane per staged row plus the checking lane");
  static_assert((ROWS & (ROWS - 1)) == 0, "full blocks split piece indexes with shifts");
  __shared__ long long s_off[ROWS];   // source byte offset of each staged row, -1 = zero row
  __shared__ int s_ok, s_nt;
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
        latch_gather(g.ctr, ULA_ENOTRESIDENT);
        ok = 0;
      }
      s_ok = ok;
      // the load hint: a one-layer gather of the step's own selection, which
      // repeats no entry (a hint only: either kind of load reads the same bytes)
      s_nt = g.Lg == 1 && n == n_res && g.ctr->res_dup[want_flag & 1] == 0;
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
    // 2. stream the staged rows (one layer: no layer arithmetic per piece)
    const int nrows = min(ROWS, n - row0);
    vec4u* o = reinterpret_cast<vec4u*>(out) + (size_t)row0 * C;
    if (nl == 1) {   // kernel-uniform
      if (s_nt)      // block-uniform
        stream_rows<ROWS, UNROLL, THREADS, false, true>(g, s_off, nrows, 1, 0, o, C, per_row);
      else
        stream_rows<ROWS, UNROLL, THREADS, false, false>(g, s_off, nrows, 1, 0, o, C, per_row);
    } else {
      stream_rows<ROWS, UNROLL, THREADS, true, false>(g, s_off, nrows, nl, layer_stride, o, C, per_row);
    }
    __syncthreads();
  }
  if (err) latch_gather(g.ctr, err);
}

template <int ROWS, int UNROLL, int THREADS>
static hipError_t launch_tiled(const GroupDev& g, const int32_t* sel, int32_t n, int32_t layer, int32_t nl,
                               uint8_t* out, long long want_flag, int32_t n_res, hipStream_t s,
                               hipEvent_t start, hipEvent_t stop) {
  int blocks = (n + ROWS - 1) / ROWS;
  if (blocks > 32768) blocks = 32768;
  const uint32_t C = (uint32_t)g.row_bytes / 16u;
  const size_t layer_stride = (size_t)n * C;
  const FastDiv per_row(C);
  if (start)
    hipExtLaunchKernelGGL(k_gather<ROWS, UNROLL, THREADS>, dim3(blocks), dim3(THREADS), 0, s, start, stop, 0,
                          g, sel, n, layer, nl, layer_stride, out, want_flag, n_res, per_row);
  else
    k_gather<ROWS, UNROLL, THREADS><<<blocks, THREADS, 0, s>>>(g, sel, n, layer, nl, layer_stride, out,
                                                               want_flag, n_res, per_row);
  return hipGetLastError();
}

hipError_t launch_gather(const GroupDev& g, const int32_t* sel, int32_t n, int32_t layer, int32_t nl,
                         uint8_t* out, long long want_flag, int32_t n_res, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop) {
  if (n <= 0 || nl <= 0) return hipSuccess;
  if (nl == 1 && n <= kSmallGatherRows)
    return launch_tiled<64, 11, 256>(g, sel, n, layer, nl, out, want_flag, n_res, s, start, stop);
  if (nl == 2 && (int64_t)n * nl <= 2 * kSmallGatherRows)
    return launch_tiled<32, 11, 256>(g, sel, n, layer, nl, out, want_flag, n_res, s, start, stop);
  if (nl > 2 && (int64_t)n * nl <= 2 * kSmallGatherRows)
    return launch_tiled<16, 11, 256>(g, sel, n, layer, nl, out, want_flag, n_res, s, start, stop);
  return launch_tiled<32, 3, 512>(g, sel, n, layer, nl, out, want_flag, n_res, s, start, stop);
}

}  // namespace ula
