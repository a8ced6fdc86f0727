// Device generator of synthetic KV rows (inputs only; no part of the engine).
//
// Row (g, la, l) is the little-endian bytes of splitmix64(x_q), q = 0 ..
// row_bytes/8 - 1, x_q = (seed << 56) ^ (g << 47) ^ (l << 39) ^ (la << 7) ^ q.
// splitmix64 is the output function of Steele, Lea and Flood (OOPSLA 2014) in
// the form Vigna publishes with xoshiro: add the golden-ratio increment, then
// two xor-shift-multiply rounds and a final xor-shift, modulo 2^64.
// out is n x layers x row_bytes bytes for the addresses las[0..n).
#include <hip/hip_runtime.h>
#include <stdint.h>

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void k_fill_rows(uint64_t* __restrict__ out, const int32_t* __restrict__ las, int64_t n,
                            int32_t layers, int32_t words, uint64_t hi) {
  const int64_t per_la = (int64_t)layers * words;
  const int64_t total = n * per_la;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_la;
    const int64_t rem = i - r * per_la;
    const uint64_t l = (uint64_t)(rem / words);
    const uint64_t q = (uint64_t)(rem - (int64_t)l * words);
    const uint64_t la = (uint64_t)(uint32_t)las[r];
    out[i] = splitmix64(hi ^ (l << 39) ^ (la << 7) ^ q);
  }
}

extern "C" int ulasynth_fill_rows(void* out_dev, const int32_t* las_dev, int64_t n, int32_t layers,
                                  int32_t row_bytes, int32_t seed, int32_t group, uint64_t stream) {
  if (n < 0 || layers < 1 || layers > 256 || row_bytes % 8 || row_bytes <= 0 || row_bytes > 1024 ||
      seed < 0 || seed > 255 || group < 0 || group > 255)
    return -1;
  if (n == 0) return 0;
  const uint64_t hi = ((uint64_t)seed << 56) ^ ((uint64_t)group << 47);
  const int64_t total = n * layers * (row_bytes / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  k_fill_rows<<<(unsigned)blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      static_cast<uint64_t*>(out_dev), las_dev, n, layers, row_bytes / 8, hi);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
