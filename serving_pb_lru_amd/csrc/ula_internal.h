// Internal layout and kernel interfaces of the PB-LRU residency engine (gfx950).
//
// One layer group owns, inside the caller's device workspace:
//   map    u32[N]        logical -> physical (GPU slot, 0x80000000|host slot, or absent)
//   tag    u64[N]        de-duplication scratch: (step << 32) | ~position, max wins
//   gown   i32[P]        owner address of each GPU slot, -1 = empty
//   stamp  i32[32 W]     step that last hit the slot (0 = never); the slots with
//                        stamp == t are the hits of step t. Padded to whole
//                        32-slot words (padding stays 0) so a lane reads one
//                        word's 32 stamps as eight 16-byte loads
//   dirty  i32[T]        step that last had a hit in each 2048-slot span
//   hown   i32[H]        owner address of each host slot, -1 = empty
//   bm     u32[NB][W]    bucket bitmaps, NB = B + 2: free, cold, ring[0..B-1]
//   tcnt   u32[NB][T]    summary level 1: set bits per 2048-slot span (64 words,
//                        one wavefront load) of each bucket, kept exact
//   hbm    u32[WH]       free host slots bitmap, htcnt u32[TH] its span counts
//   lists  hit slots, misses (address, host slot, first entry), victims, block
//          sums, work items, per-block bucket-count deltas of the mark kernel
//   res    the step's selection resolved to GPU slots, entry by entry, so that
//          every per-layer gather reads slots sequentially instead of looking
//          each address up in the mapping table again
//   stage  append addresses, destinations and (host-sourced) rows; missed rows
//          prefetched into HBM; evicted rows awaiting their write-back to the
//          host, with their host slots, and per host slot the step and staging
//          row of the last row evicted into it
//   pool   u8[P][Lg][row_bytes]   the GPU pool, slot-major: one slot holds all
//                        layers of its group contiguously
// The host pool is u8[H][Lg][row_bytes] per group in pinned, device-mapped memory.
// All groups' counters sit in one array at the front of the workspace.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ula.h"

namespace ula {

constexpr uint32_t kAbsent = 0xFFFFFFFFu;
constexpr long long kFlagFailed = 1ll << 62;    // completion counter: a step failed on the device
constexpr uint32_t kHostBit = 0x80000000u;
constexpr int kWave = 64;
constexpr int kTileWords = 64;                  // bitmap words per summary span
constexpr int kTileShift = 11;                  // 2048 slots per span
constexpr int kScanBlock = 1024;                // selection entries per de-dup block
constexpr int kMaxRing = 64;                    // B <= 64
constexpr int kMaxBuckets = kMaxRing + 2;
constexpr int kMarkBlocks = 32;                 // mark workgroups (1024 threads each) of the mark kernel
constexpr int kPrefetchBlocks = 32;             // its prefetch workgroups (missed rows into HBM)
constexpr int kWritebackBlocks = 16;            // its write-back workgroups (last step's evictions out)
constexpr int64_t kInterleavedLinkBytes = 4ll << 20;   // from this many bytes in a direction, every link
                                                        // workgroup moves both directions
constexpr int kExtractHelpers = 8;              // its extraction workgroups (besides the planning one)

// bucket ids
constexpr int kFree = 0;
constexpr int kCold = 1;
__host__ __device__ constexpr int ring_id(int b) { return 2 + b; }

struct alignas(64) Counters {
  int32_t status;        // first latched device error of the group's steps, 0 = none
  int32_t gstatus;       // first device error a gather of the group found (kept apart
                         //   from status: the step kernels poll status only, so a
                         //   gather issued out of order cannot stop a step half-way)
  long long flag;        // completion counter: last completed step
  long long stats[6];    // unique, hits, misses, evictions, from_free, invalid
  int32_t n_unique, n_hits, n_miss, n_invalid;
  int32_t n_items;       // work items written by the last selection plan
  int32_t hfree;         // free host slots
  int32_t bcnt[kMaxBuckets];  // slots per bucket
  int32_t wb_n;          // pairs of the last swap, for the deferred write-back of its victims
  int32_t done_mark;     // ticket of the mark kernel's last-workgroup plan
  int32_t lb_ticket;     // order in which compaction workgroups start (look-back scan)
  int32_t pad_acc;       // padding entries counted by the tag kernel
  uint32_t wb_step;      // step whose swap staged the rows in evict_rows (0 = none)
  int32_t mark_role;     // order in which the mark launch's workgroups start (their roles)
  uint32_t plan_done;    // step whose victim plan is published (extraction may start)
  // exact-LRU selection (policy ULA_POLICY_LRU)
  uint32_t lru_prefix;   // high key bits fixed by the select passes so far
  int32_t lru_below;     // candidate slots whose key lies below that prefix
  int32_t lru_nfree;     // free slots seen by the first select pass
  int32_t lru_ticket;    // last-workgroup ticket of the select, count and sort-count kernels
  uint32_t lru_kstar;    // key of the last victim
  int32_t lru_c;         // victims with a key below it (they need sorting by key)
  int32_t lru_r;         // victims with that key (taken in slot order)
  // first span of the free GPU set / free host set that may hold a set bit: both
  // are taken lowest first, so every span before the hint is empty (a freed host
  // slot lowers its hint)
  int32_t free_lo, hfree_lo;
  // an append under ULA_PLACE_RING: GPU slots it took, of which free ones
  int32_t app_q, app_qfree;
  // entries of a step's selection that repeat an earlier one (padding aside), by
  // step parity: a gather of that selection with none reads its rows once
  int32_t res_dup[2];
};
static_assert(sizeof(Counters) % 64 == 0, "counter block alignment");

struct SelItem {         // one summary span of one bitmap to extract set bits from
  int32_t src;           // bucket id, or kHostFreeId for the free-host bitmap
  int32_t tile;          // span index
  int32_t out_off;       // rank of the span's first taken bit in the output list
  int32_t take;          // how many of its lowest set bits to take
};
constexpr int kHostFreeId = kMaxBuckets;

struct GroupDev {        // device view of one group, passed by value to kernels
  Counters* ctr;
  uint32_t* map;
  unsigned long long* tag;
  int32_t* gown;
  int32_t* stamp;
  int32_t* dirty;
  int32_t* hown;
  uint32_t* bm;
  uint32_t* tcnt;
  uint32_t* hbm;
  uint32_t* htcnt;
  uint32_t* hit_slots;
  int32_t* miss_la;
  uint32_t* miss_h;
  int32_t* miss_e;       // [maxU] selection entry of each miss's first occurrence
  uint32_t* miss_stage;  // [maxU] staging row of the previous step holding the missed row, or absent
  uint8_t* miss_rows;    // [maxU][slot_bytes] missed rows prefetched into HBM
  unsigned long long* hs_stage;  // [H] (step << 32) | staging row of the row last evicted into
                                 //   each host slot (until that step's write-back lands)
  uint2* res;            // [max_sets * max_k] per selection entry of the last step:
                         //   (address, GPU slot), or (address, 0x80000000 | entry of the
                         //   first occurrence) for a repeated miss; (-1, absent) for padding
  uint32_t* victims;
  unsigned long long* desc;  // [2][maxBlk] look-back descriptors of the compaction, by step parity
  int32_t* partial;      // [kMarkBlocks][kMaxBuckets] bucket-count deltas of the mark kernel
  SelItem* items;
  int32_t* app_la;
  uint32_t* app_dst;
  uint8_t* app_rows;
  uint8_t* evict_rows;   // [maxU][slot_bytes] evicted rows staged for the write-back
  uint32_t* wb_h;        // [maxU] host slot each staged row goes to, or absent
  // exact-LRU state and scratch (allocated only for that policy)
  int32_t* lru_ts;       // [32 W] timestamp of each slot (hit or load step; 0 = never), written
                         //   only by the commit, so a failed step leaves it unchanged
  uint32_t* lru_hist;    // [2048] histogram of one select pass
  uint32_t* span_a;      // [T] per 2048-slot span: victims below the last key, then their offsets
  uint32_t* span_b;      // [T] per span: slots with the last key, then their offsets
  uint32_t* sort_key[2]; // [maxU] keys of the victims below the last key, ping-pong
  uint32_t* sort_slot[2];// [maxU] their slots
  uint32_t* rs_hist;     // [256][maxRs] per-block digit counts of a sort pass, then offsets
  uint32_t* rs_base;     // [256] first position of each digit
  uint8_t* pool;
  uint8_t* host;
  int32_t N, P, H, B, NB, W, T, WH, TH, Lg, row_bytes, slot_bytes;
  int32_t policy;        // ULA_POLICY_PBLRU or ULA_POLICY_LRU
  int32_t maxRs;         // sort blocks of 1024 victims
  int32_t maxU, maxBlk;  // capacity of the hit / miss / victim lists; compaction workgroups
};

// unsigned division by a run-time constant d (1 <= d < 2^31) for n < 2^31:
// q = (umulhi(m, n) + n) >> l with l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1
// (Granlund and Montgomery, "Division by invariant integers using multiplication", 1994)
struct FastDiv {
  uint32_t d, m, l;
  __host__ FastDiv() : d(1), m(1), l(0) {}
  __host__ explicit FastDiv(uint32_t div) : d(div) {
    l = 0;
    while ((1ull << l) < div) ++l;
    m = (uint32_t)(((1ull << 32) * ((1ull << l) - div)) / div + 1);
  }
  __host__ __device__ inline uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t t = __umulhi(m, n);
#else
    uint32_t t = (uint32_t)(((uint64_t)m * n) >> 32);
#endif
    return (t + n) >> l;
  }
};

// kPlanAppend: appends into free GPU slots (joining cold), then free host slots.
// kPlanAppendRing: appends into the step's victim order (free, cold, ring oldest
// to newest, never the current bucket), joining the current bucket; then free
// host slots for the entries they displace and for the entries left over.
enum PlanMode : int32_t { kPlanStep = 0, kPlanAppend = 1, kPlanAppendRing = 2 };

struct PlanArgs {
  int32_t mode;
  int32_t n;             // append: entries to place
  int32_t norder;
  int32_t dest;          // bucket the taken GPU slots join
  int8_t order[kMaxBuckets + 1];
};

// Appends of up to small_append_limit(policy) entries run as one workgroup (in the
// step's first launch under ula_append_step); larger ones through the
// multi-workgroup plan / extract / place kernels. Under PB-LRU the limit is 128:
// the multi-workgroup kernels place 256 rows per group step faster than the one
// workgroup, which the step's first launch would wait for. Under exact LRU it is
// 256: its step already has more launches in a row after the host link, and three
// more launches before the step cost it more than the one workgroup does.
constexpr int kSmallAppend = 256;   // the most entries one workgroup places
inline int small_append_limit(int policy) { return policy == ULA_POLICY_LRU ? kSmallAppend : 128; }

struct SmallAppend {
  int32_t n;
  int32_t ring;          // 1: placement into the current bucket (ULA_PLACE_RING)
  int32_t cur;           // the current bucket (placement ring)
  int32_t las[kSmallAppend];
};

// The plan of an append of n entries under ULA_PLACE_RING with current bucket
// cur: the step's victim sources in order, then the free host slots.
__host__ __device__ inline PlanArgs ring_append_plan(int32_t n, int32_t cur, int32_t B) {
  PlanArgs a{};
  a.mode = kPlanAppendRing;
  a.n = n;
  a.dest = ring_id(cur);
  a.order[0] = kFree;
  a.order[1] = kCold;
  a.norder = 2;
  for (int j = 1; j < B; ++j) a.order[a.norder++] = (int8_t)ring_id((cur + j) % B);
  a.order[a.norder++] = (int8_t)kHostFreeId;
  return a;
}

// ---- launchers (one translation unit per kernel family) ----------------
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
hipError_t launch_fill_u64(unsigned long long* p, size_t n, unsigned long long v, hipStream_t s);
hipError_t launch_init_bitmap(uint32_t* words, int32_t nwords, int64_t nbits, uint32_t* tcnt,
                              int32_t ntiles, hipStream_t s);
hipError_t launch_init_counters(Counters* c, int32_t P, int32_t H, hipStream_t s);

hipError_t launch_tag(const GroupDev& g, const int32_t* sel, int32_t n, uint32_t t, hipStream_t s);
// start / stop (both or neither): events the launch records in its own dispatch
hipError_t launch_mark(const GroupDev& g, uint32_t t, int32_t cur, const PlanArgs& a,
                       int32_t max_pairs, int32_t wb_pairs, hipStream_t s, hipEvent_t start,
                       hipEvent_t stop);
hipError_t launch_compact(const GroupDev& g, const int32_t* sel, int32_t n, uint32_t t, hipStream_t s);
hipError_t launch_plan(const GroupDev& g, const PlanArgs& a, hipStream_t s);
hipError_t launch_extract(const GroupDev& g, int32_t mode, int32_t dest, int32_t max_items,
                          hipStream_t s);
hipError_t launch_append_small(const GroupDev& g, const SmallAppend& a, const uint8_t* rows,
                              hipStream_t s);
// the step's tag pass with a small append in the same launch (ula_append_step)
hipError_t launch_tag_append(const GroupDev& g, const SmallAppend& a, const uint8_t* rows,
                             const int32_t* sel, int32_t n, uint32_t t, hipStream_t s);
hipError_t launch_place(const GroupDev& g, int32_t n, const uint8_t* rows, hipStream_t s);
hipError_t launch_place_ring(const GroupDev& g, int32_t n, const uint8_t* rows, hipStream_t s);
hipError_t launch_release(const GroupDev& g, int32_t n, hipStream_t s);
hipError_t launch_swap_commit(const GroupDev& g, uint32_t t, int32_t max_pairs, hipStream_t s);
hipError_t launch_writeback(const GroupDev& g, int32_t max_pairs, hipStream_t s);
// exact-LRU victim selection (k_lru.hip)
hipError_t launch_lru_select(const GroupDev& g, uint32_t t, int32_t max_pairs, int32_t wb_pairs,
                             hipStream_t s, hipEvent_t start, hipEvent_t stop);
hipError_t launch_lru_order(const GroupDev& g, uint32_t t, int32_t max_pairs, hipStream_t s);

// start / stop (both or neither): events recorded by the dispatch itself, so
// that their interval is the kernel's execution
// layers layer .. layer + nl - 1, each into its own n-row buffer, one after
// the other from out
hipError_t launch_gather(const GroupDev& g, const int32_t* sel, int32_t n, int32_t layer, int32_t nl,
                         uint8_t* out, long long want_flag, int32_t n_res, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop);

}  // namespace ula
