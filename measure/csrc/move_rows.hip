// Plain row moves for measurement probes: the rows, sizes and access pattern of the
// engine's miss path (random host slots <-> contiguous HBM) and of its gather (random
// HBM slots -> contiguous HBM), each direction a launch of its own with nothing else in
// it, so the engine's fused kernels can be set against the plain form and against the
// copy engines. Not part of the engine.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t vec4u __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte pieces in flight per lane

// SCATTER = false: row r of dst = row idx[r] of src (a gather: random reads,
// contiguous writes). SCATTER = true: row idx[r] of dst = row r of src (random
// writes). Lane i of a round takes piece (i mod C) of row (i div C), so
// consecutive lanes move consecutive 16 bytes of one row; non-temporal stores, and
// non-temporal loads when NT.
template <bool SCATTER, bool NT>
__global__ __launch_bounds__(kThreads) void k_move_rows(const uint8_t* __restrict__ src,
                                                       const uint32_t* __restrict__ idx,
                                                       uint8_t* __restrict__ dst, uint32_t n, uint32_t C,
                                                       uint32_t row_bytes) {
  const uint32_t total = n * C;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t base = blockIdx.x * kThreads + threadIdx.x; base < total; base += stride * kUnroll) {
    vec4u v[kUnroll];
    vec4u* d[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t i = base + u * stride;
      d[u] = nullptr;
      if (i < total) {
        const uint32_t r = i / C;
        const uint32_t c = i - r * C;
        const size_t from = SCATTER ? r : idx[r];
        const size_t to = SCATTER ? idx[r] : r;
        const vec4u* p = reinterpret_cast<const vec4u*>(src + from * row_bytes) + c;
        v[u] = NT ? __builtin_nontemporal_load(p) : *p;
        d[u] = reinterpret_cast<vec4u*>(dst + to * row_bytes) + c;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (d[u]) __builtin_nontemporal_store(v[u], d[u]);
  }
}

// A contiguous device copy of `pieces` 16-byte pieces: the plain form of the
// gather's HBM traffic with no row indexing at all. Each workgroup takes
// kThreads * kUnroll consecutive pieces per round (grid-stride over rounds),
// kUnroll in flight per lane; non-temporal stores, and non-temporal loads when NT
// (a copy reads its source once, as the gather of a step without repeats does).
template <bool NT>
__global__ __launch_bounds__(kThreads) void k_copy(const vec4u* __restrict__ src, vec4u* __restrict__ dst,
                                                  uint32_t pieces) {
  const uint32_t chunk = kThreads * kUnroll;
  for (uint32_t base = blockIdx.x * chunk + threadIdx.x; base < pieces; base += gridDim.x * chunk) {
    vec4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t i = base + u * kThreads;
      if (i < pieces) v[u] = NT ? __builtin_nontemporal_load(src + i) : src[i];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t i = base + u * kThreads;
      if (i < pieces) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

}  // namespace

// mode 0: gather, dst[r] = src[idx[r]] for r < n; mode 1: scatter, dst[idx[r]] = src[r];
// mode 2: the gather with non-temporal loads.
// src, idx, dst: device pointers or pinned host pointers the device can reach;
// rows are row_bytes apart (a multiple of 16). Every idx[r] must be a row of the
// buffer it indexes (the caller checks; the kernel does not). blocks: workgroups of
// 256 lanes (grid-stride). Returns 0, -1 for bad arguments, -2 if the launch failed.
extern "C" int probe_move_rows(int mode, const void* src, const uint32_t* idx, void* dst, uint32_t n,
                              uint32_t row_bytes, int blocks, uint64_t stream) {
  if (mode < 0 || mode > 2 || !src || !idx || !dst || row_bytes == 0 || row_bytes % 16 || blocks < 1 ||
      blocks > (1 << 20))
    return -1;
  const uint32_t C = row_bytes / 16;
  if ((uint64_t)n * C + (uint64_t)blocks * kThreads * kUnroll >= (1ull << 32)) return -1;
  if (n == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* a = static_cast<const uint8_t*>(src);
  uint8_t* b = static_cast<uint8_t*>(dst);
  if (mode == 0)
    k_move_rows<false, false><<<blocks, kThreads, 0, s>>>(a, idx, b, n, C, row_bytes);
  else if (mode == 2)
    k_move_rows<false, true><<<blocks, kThreads, 0, s>>>(a, idx, b, n, C, row_bytes);
  else
    k_move_rows<true, false><<<blocks, kThreads, 0, s>>>(a, idx, b, n, C, row_bytes);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// dst[0, nbytes) = src[0, nbytes): device pointers, 16-byte aligned, nbytes a multiple
// of 16. blocks: workgroups of 256 lanes (grid-stride); nt: non-temporal loads.
// Returns 0, -1 for bad arguments, -2 if the launch failed.
extern "C" int probe_copy(const void* src, void* dst, uint64_t nbytes, int blocks, int nt, uint64_t stream) {
  if (!src || !dst || nbytes % 16 || blocks < 1 || blocks > (1 << 20) ||
      ((uintptr_t)src | (uintptr_t)dst) % 16)
    return -1;
  const uint64_t pieces = nbytes / 16;
  if (pieces + (uint64_t)blocks * kThreads * kUnroll >= (1ull << 32)) return -1;
  if (pieces == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (nt)
    k_copy<true><<<blocks, kThreads, 0, s>>>(static_cast<const vec4u*>(src), static_cast<vec4u*>(dst),
                                             (uint32_t)pieces);
  else
    k_copy<false><<<blocks, kThreads, 0, s>>>(static_cast<const vec4u*>(src), static_cast<vec4u*>(dst),
                                              (uint32_t)pieces);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
