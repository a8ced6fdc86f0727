// The de-duplication tag pass, shared by the tag kernel and the launch that
// also carries a step's small append.
//
// UlaCache summary (paper-daily.com), section 2: the layers sharing a selection
// look it up and de-duplicate it once per group. Every in-range entry e of the
// step's selection stores key(t, e) = (t << 32) | ~e into tag[la] with a 64-bit
// atomic max, so once the pass has completed tag[la] holds the key of la's
// first occurrence in step t (a smaller e gives a larger ~e; tags of earlier
// steps have a smaller t and never match). An address outside [0, N) is an
// error; one never appended is found by the compaction, which reads the
// mapping table anyway (so this pass reads only the selection and may run
// beside an append).
#pragma once

#include "device_util.h"

namespace ula {

__device__ __forceinline__ unsigned long long dedup_key(uint32_t t, uint32_t e) {
  return ((unsigned long long)t << 32) | (unsigned long long)(~e);
}

// Workgroup `part` of `nparts` (any block size). Also clears the look-back
// descriptors of parity t & 1, which the step's compaction uses (their last
// user, the step before the previous one, has completed), and counts padding.
// No error check up front: this pass writes only scratch (tags, descriptors,
// the padding count), and a latched error stops the compaction, which is where
// the step's results are written.
__device__ __forceinline__ void tag_entries(const GroupDev& g, const int32_t* __restrict__ sel, int32_t n,
                                            uint32_t t, int part, int nparts) {
  const int stride = nparts * blockDim.x;
  unsigned long long* desc = g.desc + (size_t)(t & 1u) * g.maxBlk;
  for (int i = part * blockDim.x + threadIdx.x; i < g.maxBlk; i += stride) desc[i] = 0ull;
  bool bad = false;
  int pad = 0;
  for (int e = part * blockDim.x + threadIdx.x; e < n; e += stride) {
    const int32_t la = sel[e];
    if (la == -1) {
      ++pad;
      continue;
    }
    if (la < 0 || la >= g.N) {
      bad = true;
      continue;
    }
    atomicMax(&g.tag[la], dedup_key(t, (uint32_t)e));
  }
  if (bad) latch(g.ctr, ULA_ERANGE);
  // padding entries of the step (statistics); one atomic per wavefront that saw any
  pad = wave_sum(pad);
  if (pad && lane_id() == 0) atomicAdd(&g.ctr->pad_acc, pad);
}

}  // namespace ula
