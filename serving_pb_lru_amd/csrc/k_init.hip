// Initialisation kernels: fills, bitmaps with their span counts, counters.
// Plain fill kernels are used instead of hipMemsetAsync so that the whole
// initialisation is ordinary kernel work on the caller's stream.
#include "device_util.h"

namespace ula {

__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void k_fill_u64(unsigned long long* p, size_t n, unsigned long long v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Set bits [0, nbits) of a bitmap of nwords words, clear the rest, and write
// the population count of every 64-word span. One wavefront per span.
__global__ void k_init_bitmap(uint32_t* words, int32_t nwords, int64_t nbits, uint32_t* tcnt,
                              int32_t ntiles) {
  const int lane = lane_id();
  const int nwaves = gridDim.x * (blockDim.x / kWave);
  for (int tile = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; tile < ntiles;
       tile += nwaves) {
    int w = tile * kTileWords + lane;
    uint32_t x = 0;
    if (w < nwords) {
      int64_t lo = (int64_t)w * 32;
      if (lo + 32 <= nbits) x = 0xFFFFFFFFu;
      else if (lo < nbits) x = (1u << (uint32_t)(nbits - lo)) - 1u;
      words[w] = x;
    }
    int c = wave_inclusive_sum(__popc(x));
    if (lane == kWave - 1) tcnt[tile] = (uint32_t)c;
  }
}

// Every field starts at zero (one lane per 32-bit word of the block, so that
// no field can be left uninitialised), then the non-zero ones are set.
__global__ void k_init_counters(Counters* c, int32_t P, int32_t H) {
  uint32_t* words = reinterpret_cast<uint32_t*>(c);
  for (int i = threadIdx.x; i < (int)(sizeof(Counters) / 4); i += blockDim.x) words[i] = 0u;
  __syncthreads();
  if (threadIdx.x != 0) return;
  c->hfree = H;
  c->bcnt[kFree] = P;
}

static int grid_for(size_t n, int bs) {
  size_t b = (n + bs - 1) / bs;
  return (int)(b < 4096 ? (b ? b : 1) : 4096);
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
  if (!n) return hipSuccess;
  k_fill_u32<<<grid_for(n, 256), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_u64(unsigned long long* p, size_t n, unsigned long long v, hipStream_t s) {
  if (!n) return hipSuccess;
  k_fill_u64<<<grid_for(n, 256), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_init_bitmap(uint32_t* words, int32_t nwords, int64_t nbits, uint32_t* tcnt,
                              int32_t ntiles, hipStream_t s) {
  if (!ntiles) return hipSuccess;
  int blocks = (ntiles + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  k_init_bitmap<<<blocks, 256, 0, s>>>(words, nwords, nbits, tcnt, ntiles);
  return hipGetLastError();
}

hipError_t launch_init_counters(Counters* c, int32_t P, int32_t H, hipStream_t s) {
  k_init_counters<<<1, 64, 0, s>>>(c, P, H);
  return hipGetLastError();
}

}  // namespace ula
