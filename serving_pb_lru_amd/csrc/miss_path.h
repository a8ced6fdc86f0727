// Host-link parts of the miss path, shared by the mark kernel (which runs them
// in extra workgroups beside the hit marking) and the stand-alone write-back.
//
// UlaCache summary (paper-daily.com), section 3: data moves before the
// mapping changes; section 2: an entry lives in exactly one pool. Pair i of a
// step brings the missed entry miss_la[i] in from host slot miss_h[i] and sends
// the entry of its victim slot out to that same host slot.
//
// The host pool is pinned, device-mapped memory read and written directly with
// 16-byte vector accesses. Both directions of the link run at once: a step's
// prefetch reads its missed rows while the previous step's evicted rows are
// written out. The two never touch the same host slot: a slot written by the
// write-back of step t - 1 holds an entry evicted by step t - 1, and a miss of
// that entry in step t reads the staged copy instead (miss_stage).
#pragma once

#include "device_util.h"

namespace ula {

// Stores to the host pool are non-temporal: measured against plain stores of
// the same bytes, the default workload's link phase went from 66-67 to 61-63
// us and the speculative workload's steps became 3% shorter; the eviction
// control and the eviction-heavy workload did not change.
//
// Request depth. In the two loops below each of a lane's U pieces first loads a
// small record (staging row or host slot) and then its data; loads complete in
// order, so each record load also waits for the previous piece's host access,
// and a lane keeps about one host request in flight. That depth is deliberate:
// issuing every piece's records first and then all U host reads together (U
// host reads in flight per lane) made the default workload's link phase 7%
// slower and the eviction-heavy one 9% slower, with the same link bytes. The
// interleaved loop further below keeps one piece per direction in flight too,
// but loads the next piece's records while the current piece's data is on its
// way (the eviction-heavy workload's link launch 4.09 -> 3.98 ms); the same in
// these two loops changed the one-group workload's steps by less than 1%.

// Missed rows of step t (all layers, one contiguous slot_bytes run each) into
// miss_rows[i], from the host pool or from the staging copy of step t - 1. m is
// the step's miss count (the caller loads it with its other first loads).
// Workgroup `part` of `nparts`, blockDim.x threads each.
__device__ __forceinline__ void prefetch_misses(const GroupDev& g, int m, FastDiv per_slot, int part,
                                                int nparts) {
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t total = (uint32_t)m * chunks;
  const uint32_t stride = (uint32_t)nparts * blockDim.x;
  constexpr int U = 4;
  for (uint32_t base = (uint32_t)part * blockDim.x + threadIdx.x; base < total; base += U * stride) {
    vec4u v[U];
    vec4u* dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + u * stride;
      dst[u] = nullptr;
      if (idx < total) {
        const uint32_t i = per_slot.div(idx);
        const uint32_t c = idx - i * chunks;
        const uint32_t from = g.miss_stage[i];
        const uint8_t* src = from != kAbsent ? g.evict_rows + (size_t)from * g.slot_bytes
                                             : g.host + (size_t)g.miss_h[i] * g.slot_bytes;
        v[u] = reinterpret_cast<const vec4u*>(src)[c];
        dst[u] = reinterpret_cast<vec4u*>(g.miss_rows + (size_t)i * g.slot_bytes) + c;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst[u]) *dst[u] = v[u];
  }
}

// The rows staged by the swap of step `t` go to the host slots their misses
// vacated (wb_h; absent for a victim that was free). staged_step and staged_n
// are the counter block's record of what the staging buffer holds (the caller
// loads them with its other first loads); nothing happens unless it holds
// step t's rows.
__device__ __forceinline__ void writeback_rows(const GroupDev& g, uint32_t staged_step, int staged_n,
                                               uint32_t t, FastDiv per_slot, int part, int nparts) {
  if (staged_step != t) return;
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t total = (uint32_t)staged_n * chunks;
  const uint32_t stride = (uint32_t)nparts * blockDim.x;
  constexpr int U = 2;   // pieces per lane and round (measured: 1% faster steps than 4 or 8)
  for (uint32_t base = (uint32_t)part * blockDim.x + threadIdx.x; base < total; base += U * stride) {
    vec4u v[U];
    vec4u* hp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + u * stride;
      hp[u] = nullptr;
      if (idx < total) {
        const uint32_t i = per_slot.div(idx);
        const uint32_t c = idx - i * chunks;
        const uint32_t h = g.wb_h[i];
        if (h != kAbsent) {
          hp[u] = reinterpret_cast<vec4u*>(g.host + (size_t)h * g.slot_bytes) + c;
          v[u] = reinterpret_cast<const vec4u*>(g.evict_rows + (size_t)i * g.slot_bytes)[c];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (hp[u]) __builtin_nontemporal_store(v[u], hp[u]);
  }
}

// Both directions in every link workgroup: each iteration loads a piece of
// missed rows and a piece of staged rows, then stores both. m missed rows
// come in; wb_rows staged rows (0: none) go out to their host slots.
// Workgroup `part` of `nparts`.
__device__ __forceinline__ void swap_rows_interleaved(const GroupDev& g, int m, int wb_rows, FastDiv per_slot,
                                                      int part, int nparts) {
  const uint32_t chunks = (uint32_t)g.slot_bytes / 16u;
  const uint32_t tp = (uint32_t)m * chunks;
  const uint32_t tw = (uint32_t)wb_rows * chunks;
  const uint32_t total = tp > tw ? tp : tw;
  const uint32_t stride = (uint32_t)nparts * blockDim.x;
  // The records of a lane's next piece (staging row and host slot of its miss,
  // host slot of its write-back) are loaded while its current piece's data is in
  // flight, so a piece waits only for its data. One piece per direction and lane
  // is in flight: two, with both pieces' records loaded ahead, measured 0-1%
  // slower (the eviction workload, its control, six groups of the 24-group one).
  uint32_t from = kAbsent, mh = 0, h = kAbsent;
  uint32_t base = (uint32_t)part * blockDim.x + threadIdx.x;
  if (base < tp) {
    const uint32_t i = per_slot.div(base);
    from = g.miss_stage[i];
    mh = g.miss_h[i];
  }
  if (base < tw) h = g.wb_h[per_slot.div(base)];
  for (; base < total; base += stride) {
    vec4u pv, wv;
    vec4u* pd = nullptr;
    vec4u* wd = nullptr;
    if (base < tp) {
      const uint32_t i = per_slot.div(base);
      const uint32_t c = base - i * chunks;
      const uint8_t* src = from != kAbsent ? g.evict_rows + (size_t)from * g.slot_bytes
                                           : g.host + (size_t)mh * g.slot_bytes;
      pv = reinterpret_cast<const vec4u*>(src)[c];
      pd = reinterpret_cast<vec4u*>(g.miss_rows + (size_t)i * g.slot_bytes) + c;
    }
    if (base < tw && h != kAbsent) {
      const uint32_t i = per_slot.div(base);
      const uint32_t c = base - i * chunks;
      wd = reinterpret_cast<vec4u*>(g.host + (size_t)h * g.slot_bytes) + c;
      wv = reinterpret_cast<const vec4u*>(g.evict_rows + (size_t)i * g.slot_bytes)[c];
    }
    const uint32_t next = base + stride;
    from = kAbsent;
    h = kAbsent;
    if (next < tp) {
      const uint32_t i = per_slot.div(next);
      from = g.miss_stage[i];
      mh = g.miss_h[i];
    }
    if (next < tw) h = g.wb_h[per_slot.div(next)];
    if (pd) *pd = pv;
    if (wd) __builtin_nontemporal_store(wv, wd);
  }
}

// The link work of a step's selection launch, workgroup `part` of its pf
// prefetch and wbb write-back workgroups (m: the step's misses; staged_step /
// staged_n: the counter block's record of the staging buffer; wb_step: the
// step whose staged rows go out, meaningful when wbb > 0). A step that moves
// at least kInterleavedLinkBytes in a direction runs both directions in every
// link workgroup; a smaller one keeps them in separate workgroups (measured:
// interleaving made the steps of the workloads moving 6-156 MB each way 1-10%
// shorter, but the default workload's 2 MB link phase 15% longer, since a
// lane's next host read then waits for its previous host write).
__device__ __forceinline__ void link_part(const GroupDev& g, int m, uint32_t staged_step, int staged_n,
                                          uint32_t wb_step, FastDiv per_slot, int part, int pf, int wbb) {
  const int wb_rows = (wbb > 0 && staged_step == wb_step) ? staged_n : 0;
  const int rows = m > wb_rows ? m : wb_rows;
  if ((int64_t)rows * g.slot_bytes >= kInterleavedLinkBytes)   // uniform over the launch
    swap_rows_interleaved(g, m, wb_rows, per_slot, part, pf + wbb);
  else if (part >= pf)
    writeback_rows(g, staged_step, staged_n, wb_step, per_slot, part - pf, wbb);
  else
    prefetch_misses(g, m, per_slot, part, pf);
}

}  // namespace ula
