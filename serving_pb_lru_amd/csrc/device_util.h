// Wavefront and workgroup primitives for gfx950 (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ula_internal.h"

namespace ula {

// 16 bytes moved as one vector access (global_load/store_dwordx4)
typedef uint32_t vec4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Number of set bits of `mask` below this lane (the lane's rank among the
// lanes whose ballot bit is set).
__device__ __forceinline__ int rank_below(unsigned long long mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int u = __shfl_up(v, d, kWave);
    if (lane_id() >= d) v += u;
  }
  return v;
}

// Sum over the 64 lanes of a wavefront, returned to every lane.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Exclusive prefix sum over a whole workgroup of NT threads; `total` receives
// the sum over the workgroup. `scratch` holds NT / 64 + 1 ints of LDS. Every thread
// of the workgroup must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int* scratch, int& total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int inc = wave_inclusive_sum(v);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < NW ? scratch[lane] : 0;
    int wi = wave_inclusive_sum(w);
    if (lane < NW) scratch[lane] = wi - w;   // exclusive wave offsets
    if (lane == NW - 1) scratch[NW] = wi;    // total
  }
  __syncthreads();
  int res = scratch[wave] + inc - v;
  total = scratch[NW];
  __syncthreads();
  return res;
}

// Latch the first device error of a group; later kernels read it and exit.
__device__ __forceinline__ void latch(Counters* c, int code) {
  atomicCAS(&c->status, 0, code);
}

// Latch the first error a gather found, apart from the steps' status.
__device__ __forceinline__ void latch_gather(Counters* c, int code) {
  atomicCAS(&c->gstatus, 0, code);
}

__device__ __forceinline__ int status_of(const Counters* c) {
  return __hip_atomic_load(&c->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-uniform error check for kernels that use workgroup barriers: every
// thread of the workgroup sees the same answer.
__device__ __forceinline__ bool block_failed(const Counters* c) {
  __shared__ int s_status;
  if (threadIdx.x == 0) s_status = status_of(c);
  __syncthreads();
  return s_status != 0;
}

__device__ __forceinline__ uint32_t* bucket_words(const GroupDev& g, int id) {
  return id == kHostFreeId ? g.hbm : g.bm + (size_t)id * g.W;
}
__device__ __forceinline__ uint32_t* bucket_tcnt(const GroupDev& g, int id) {
  return id == kHostFreeId ? g.htcnt : g.tcnt + (size_t)id * g.T;
}
__device__ __forceinline__ int bucket_nwords(const GroupDev& g, int id) {
  return id == kHostFreeId ? g.WH : g.W;
}
__device__ __forceinline__ int bucket_ntiles(const GroupDev& g, int id) {
  return id == kHostFreeId ? g.TH : g.T;
}
__device__ __forceinline__ int32_t* bucket_count(const GroupDev& g, int id) {
  return id == kHostFreeId ? &g.ctr->hfree : &g.ctr->bcnt[id];
}

// Piece c (16 bytes, value v) of appended entry `la` goes to the destination
// chosen for it (d: a GPU slot, or a host slot with the host bit); the lane of
// piece 0 also publishes the mapping and owner entries of `la`.
__device__ __forceinline__ void place_piece(const GroupDev& g, uint32_t d, uint32_t c, int32_t la,
                                            const vec4u v) {
  if (d & kHostBit)   // host pool: non-temporal, as every store to it
    __builtin_nontemporal_store(v, reinterpret_cast<vec4u*>(g.host + (size_t)(d & ~kHostBit) * g.slot_bytes) + c);
  else
    reinterpret_cast<vec4u*>(g.pool + (size_t)d * g.slot_bytes)[c] = v;
  if (c == 0) {
    g.map[la] = d;
    if (d & kHostBit) g.hown[d & ~kHostBit] = la;
    else g.gown[d] = la;
  }
}

// Piece c (16 bytes, value v) of appended entry i (address la) under
// ULA_PLACE_RING. dst holds the q GPU slots the append took (taken from the
// free set: host bit set; the first qfree of them) and then its host slots. An
// entry i < q goes to GPU slot dst[i]; the entry it displaces from an occupied
// slot first moves, rows and all, to host slot dst[q + i - qfree]. An entry
// i >= q goes to host slot dst[q + i - qfree] itself. The lane of piece 0 also
// publishes the mapping and owner entries. A piece's old row is read before
// the new one is written, by the same lane.
__device__ __forceinline__ void place_piece_ring(const GroupDev& g, const uint32_t* dst, int q, int qfree,
                                                 uint32_t i, uint32_t c, int32_t la, const vec4u v) {
  if ((int)i < q) {
    const uint32_t d = dst[i];
    const uint32_t s = d & ~kHostBit;
    vec4u* gp = reinterpret_cast<vec4u*>(g.pool + (size_t)s * g.slot_bytes) + c;
    if (!(d & kHostBit)) {   // an occupied slot: its entry moves to the host pool
      const uint32_t h = dst[q + (int)i - qfree] & ~kHostBit;
      const vec4u old = *gp;
      __builtin_nontemporal_store(old, reinterpret_cast<vec4u*>(g.host + (size_t)h * g.slot_bytes) + c);
      if (c == 0) {
        const int32_t o = g.gown[s];
        g.map[o] = kHostBit | h;
        g.hown[h] = o;
      }
    }
    *gp = v;
    if (c == 0) {
      g.map[la] = s;
      g.gown[s] = la;
    }
  } else {
    const uint32_t h = dst[q + (int)i - qfree] & ~kHostBit;
    __builtin_nontemporal_store(v, reinterpret_cast<vec4u*>(g.host + (size_t)h * g.slot_bytes) + c);
    if (c == 0) {
      g.map[la] = kHostBit | h;
      g.hown[h] = la;
    }
  }
}

}  // namespace ula
