/*
 * ula.h -- C ABI of the PB-LRU KV residency engine for MI355X (gfx950).
 *
 * The engine implements, for one GPU in data-parallel form, the residency
 * layer described in "UlaCache: Unified Logical Addressing for Sparse LLM
 * Serving" (paper-daily.com summary):
 *
 *  - Section 2: the serving engine allocates and selects KV entries by fixed
 *    logical address only; the library decides whether the GPU pool or the
 *    host pool holds each entry, moves it, and keeps a logical->physical
 *    mapping table. In DP mode an entry lives in exactly one of the two
 *    pools. Layers that share one sparse selection look up and de-duplicate
 *    it once per layer group.
 *  - Section 3: the GPU pool is managed by PB-LRU: slots are labelled with the
 *    scheduling round that last touched them (per layer group, a ring of round
 *    buckets and one cold bucket, each a bitmap with summaries); victims come
 *    from free slots, then cold, then older ring buckets, never the running
 *    round's bucket. Rows move before the mapping changes, the completion
 *    signal comes last, and readers wait for it.
 *
 * Conventions
 *  - Every layer group g in [0, num_groups) has its own GPU pool of
 *    gpu_slots slots, host pool of host_slots slots, mapping table over
 *    logical addresses [0, logical_capacity), and replacement state.
 *  - A slot holds the rows of all layers_per_group layers of one logical
 *    entry; a row is row_bytes opaque bytes (FP8 latent, rope and scales in
 *    the pages' model; never interpreted here).
 *  - Mapping table encoding (uint32): s < 2^31 = GPU slot s; 0x80000000|h =
 *    host slot h; 0xFFFFFFFF = never appended.
 *  - Bucket bitsets: words of 32 bits, slot s is bit (s & 31) of word
 *    (s >> 5); order free, cold, ring[0] .. ring[B-1].
 *  - All calls that take a stream enqueue work on that HIP stream
 *    (hipStream_t passed as uint64_t; 0 = null stream) and return without
 *    waiting, unless stated otherwise. Device-side errors of an enqueued call
 *    are reported by the next ula_sync.
 *
 * Ownership
 *  - The caller allocates and owns the device workspace (ula_device_bytes
 *    bytes, 256-byte aligned, device memory) and the pinned host pool
 *    (ula_host_bytes bytes, page-locked and device-mapped, e.g. from
 *    ula_host_alloc), the selection and output buffers and the streams. They
 *    must outlive all work enqueued on them. The library owns only the
 *    opaque context and the layout inside the two buffers.
 *
 * Errors
 *  - Every call returns ULA_OK (0) or a negative code. Errors detected on the
 *    host are returned at once and change nothing. Errors detected on the
 *    device during an enqueued step are latched per group and the remaining
 *    kernels of that step exit before changing any state; errors a gather
 *    detects are latched per group in a separate word that steps do not read,
 *    so a gather never stops a step part-way. The next ula_sync returns the
 *    first latched code and the context becomes unusable (ULA_ESTATE) for every
 *    call but ula_export_state, ula_read_rows, ula_sync and ula_destroy.
 *  - ULA_ECAPACITY is detected before any state changes, so an exported state
 *    after it is the state before the failed step.
 *
 * Threading: a context belongs to one host thread. Groups are independent and
 * may be driven on different streams; calls on one group must be ordered. The
 * groups share one host link, so once steps arrive on more than one stream the
 * library orders each step's host-link launch after the previous step's (of any
 * group) with an event; the rest of one group's step (lookup, swap, gathers)
 * still runs beside another group's host-link launch. A gather issued on a
 * stream other than its step's must be ordered after the step (an event, or a
 * stream wait on ula_flag_address). The library orders what comes after it:
 * the group's next launch that moves rows out of GPU slots (the next step's
 * swap, an append under ULA_PLACE_RING, a release) waits, by events, for the
 * group's gathers enqueued since its last such launch, on any stream; the next
 * step's lookup, marking and host-link transfers do not wait and may run beside
 * those gathers (each step resolves its selection into one of two buffers, by
 * step parity, and a gather reads its step's). HIP places a process's streams
 * on a few hardware queues, each running its launches in order: with more step
 * streams than queues, one group's lookup can wait behind another group's
 * gathers, so many groups run best on two step streams (groups alternating)
 * with the gathers on a third.
 */
#ifndef ULA_H
#define ULA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ULA_OK = 0,
  ULA_EINVAL = -1,       /* bad argument or configuration */
  ULA_ERANGE = -2,       /* logical address outside [0, N) or never appended */
  ULA_EDUP = -3,         /* append of an address already appended, or twice in one call */
  ULA_EHOSTFULL = -4,    /* no free GPU or host slot left for an append */
  ULA_ECAPACITY = -5,    /* a step selects more distinct entries than the GPU pool holds */
  ULA_ENOTRESIDENT = -6, /* gather before its step completed, or of an entry not on the GPU */
  ULA_ESTATE = -7,       /* the context was poisoned by an earlier device error */
  ULA_EHIP = -8,         /* a HIP runtime call failed; ula_strerror gives its text */
  ULA_EBUSY = -9,        /* ula_init_static: this device's static workspace is held by a live context */
  ULA_ETOOBIG = -10      /* ula_init_static: the configuration needs more than the static workspace */
};

typedef struct ula_ctx ula_ctx;

typedef struct {
  int32_t num_groups;        /* layer groups, each with its own pools and state, >= 1 */
  int32_t layers_per_group;  /* layers sharing one selection, >= 1 */
  int32_t row_bytes;         /* bytes per row, multiple of 16, <= 4096 */
  int32_t ring_buckets;      /* B >= 1 ring buckets (plus one cold and one free bucket) */
  int32_t logical_capacity;  /* N: logical addresses [0, N), 1 <= N < 2^31 */
  int32_t gpu_slots;         /* P >= 1 GPU slots per group */
  int32_t host_slots;        /* H >= 0 host slots per group, P + H < 2^31 */
  int32_t max_sets;          /* most selection sets per step */
  int32_t max_k;             /* most entries per selection set; max_sets * max_k < 2^31 */
  int32_t max_append;        /* most addresses staged per append chunk, >= 1 */
  int32_t policy;            /* ULA_POLICY_PBLRU (0, default) or ULA_POLICY_LRU (1) */
  int32_t placement;         /* where ula_append puts new entries: ULA_PLACE_LOWEST (0, default)
                                or ULA_PLACE_RING (1, PB-LRU only) */
} ula_config;

/* Placement of appended entries (section 2: the library decides which pool holds
 * new KV; the pages do not say how).
 *  - ULA_PLACE_LOWEST: in list order each entry takes the lowest free GPU slot,
 *    joining the cold bucket, else the lowest free host slot; appends never
 *    evict (with a full GPU pool, new entries start in the host pool and come
 *    in through a step's miss path when selected).
 *  - ULA_PLACE_RING: new entries count as used in the current round (section 3:
 *    recent entries stay on the GPU): in list order each entry takes the next
 *    slot of the step's victim order (free ascending, then cold, then ring
 *    buckets oldest to newest, never the current bucket) and joins the current
 *    bucket; an entry displaced from that slot moves, rows and all, to the
 *    lowest free host slot; when no such slot is left, entries take the lowest
 *    free host slots. The current bucket is that of the group's last step. */
enum { ULA_PLACE_LOWEST = 0, ULA_PLACE_RING = 1 };

/* Replacement policies. PB-LRU is the pages' policy (UlaCache summary, section 3).
 * Exact LRU is the standard policy the pages compare it against (sections 3 and 4):
 * one timestamp per GPU slot (a hit or a load at step t sets it to t; an
 * appended slot s counts as s - P, so older than any step and ordered by slot)
 * and a scan of the whole pool each step; victims are the free slots in
 * ascending order, then the occupied slots by (timestamp, slot), never a slot
 * stamped with the current step. Everything else (lookup, pairing, data moves,
 * commit, signal, appends) is shared. */
enum { ULA_POLICY_PBLRU = 0, ULA_POLICY_LRU = 1 };

typedef struct {
  int64_t unique;     /* distinct valid addresses selected by the step */
  int64_t hits;       /* of those, already on the GPU */
  int64_t misses;     /* of those, brought in from the host pool */
  int64_t evictions;  /* misses whose victim slot held an entry (sent to the host) */
  int64_t from_free;  /* misses that took a free GPU slot */
  int64_t invalid;    /* -1 padding entries in the selection */
} ula_step_stats;

typedef struct {             /* caller-allocated host buffers filled by ula_export_state */
  uint32_t* map;             /* [N] mapping table */
  int32_t* gown;             /* [P] owner logical address of each GPU slot, -1 = empty */
  int32_t* hown;             /* [H] owner logical address of each host slot, -1 = empty */
  uint32_t* bitsets;         /* [(B + 2)][ceil(P / 32)]: free, cold, ring[0..B-1]; under exact
                                LRU only the free set is kept (the others read as empty) */
  int32_t cur;               /* current ring bucket */
  int64_t flag;              /* last completed step (completion counter) */
  ula_step_stats last;       /* statistics of that step */
  int32_t* stamps;           /* nullable, [P]: exact LRU timestamps (appended slot s: s - P,
                                free slot: 0); under PB-LRU left untouched */
} ula_state_host;

/* Bytes of device workspace / pinned host pool a configuration needs; 0 for an
 * invalid configuration (section 2: in DP mode each GPU has one GPU pool and one
 * host pool; here every layer group has its own of each, plus its mapping table
 * and replacement state in the workspace). Pure host functions (no device is
 * touched). */
size_t ula_device_bytes(const ula_config* cfg);
size_t ula_host_bytes(const ula_config* cfg);

/* Lay out the workspace, initialise every group (nothing appended, all GPU slots
 * free, all host slots free, cur = 0, flag = 0) on `stream`, and return a context
 * (section 2: the pools and the mapping table; section 3: one ring plus a cold
 * bucket per layer group).
 * dev_ws: device memory of ula_device_bytes(cfg) bytes, 256-byte aligned.
 * host_pinned: pinned, device-mapped host memory of ula_host_bytes(cfg) bytes
 * (may be NULL when host_slots == 0). Errors: ULA_EINVAL, ULA_EHIP. */
int ula_init(const ula_config* cfg, void* dev_ws, void* host_pinned, uint64_t stream,
             ula_ctx** out);

/* ula_init for callers that cannot allocate device memory (code that must not
 * call hipMalloc or a caching allocator: tight serving loops, harnesses that
 * forbid allocation). Exactly ula_init, with the device workspace taken from a
 * static array the library holds on every device it runs on (32 MiB per device,
 * kept until the process ends) instead of a dev_ws argument: the current
 * device's array, resolved once per device. Only a configuration with
 * ula_device_bytes(cfg) <= 32 MiB fits (ULA_ETOOBIG otherwise, nothing
 * touched). One live context per device may hold the array: another call on the
 * same device before that context's ula_destroy returns ULA_EBUSY (two contexts
 * on one array would overwrite each other's state). Every call starts from a
 * fully initialised workspace whatever an earlier context left in it.
 * The call allocates no device memory and no pinned host memory (the context
 * itself is ordinary host memory; host_pinned is still the caller's pool). Such
 * a context has no pinned staging buffers: ula_append of more than 128 entries
 * (256 under ULA_POLICY_LRU) runs in chunks whose addresses travel by value in
 * the launches, host-resident rows are copied in and waited for chunk by chunk,
 * and ula_release copies its addresses from the caller's memory and waits for
 * that copy before it returns; the events
 * of step timing and of the ordering of host-link launches across streams are
 * created by the call that first needs them. Everything else behaves as for a
 * context from ula_init.
 * Errors: ULA_EINVAL, ULA_ETOOBIG, ULA_EBUSY, ULA_EHIP. */
int ula_init_static(const ula_config* cfg, void* host_pinned, uint64_t stream, ula_ctx** out);

/* Append n new logical entries to group g (section 2: the library decides the
 * pool), placed as the configuration's placement says: by default, in list
 * order each entry takes the lowest free GPU slot (joining the cold bucket) or,
 * when none is free, the lowest free host slot, and appends never evict; under
 * ULA_PLACE_RING each entry joins the current bucket, displacing entries to the
 * host pool (see above). la_host: n addresses in host memory. rows: n x layers_per_group x
 * row_bytes bytes, packed, in device memory (rows_on_device = 1) or host memory
 * (rows_on_device = 0); rows must stay valid until the stream reaches the call.
 * An append of more than 128 entries (256 under ULA_POLICY_LRU), or of
 * host-resident rows, copies its
 * addresses through one of four pinned staging buffers of the group: with all
 * four still in use by enqueued appends, the call first waits for the oldest to
 * be consumed (the host runs at most four such appends ahead of the device).
 * Validated on the host first: ULA_EINVAL (bad g or n < 0), ULA_ERANGE (address
 * outside [0, N)), ULA_EDUP (already appended or repeated), ULA_EHOSTFULL (not
 * enough free slots in total); nothing changes on error. */
int ula_append(ula_ctx* ctx, int32_t group, int32_t n, const int32_t* la_host,
               const void* rows, int32_t rows_on_device, uint64_t stream);

/* Release n finished entries of group g (a request has ended; section 1: in a
 * shared pool the space one request frees serves the others). Each address must
 * be appended and listed once; it becomes absent and may be appended again. Its
 * GPU slot leaves whatever bucket holds it and joins the free slots, which later
 * steps take first for their misses and appends take before host slots; or its
 * host slot joins the free host slots. The ring, the current bucket, the
 * completion counter and the statistics do not change. Staged evicted rows of
 * the last step are written to the host pool first (a released host slot may be
 * waiting for one). Gathers of the last step's selection after a release resolve
 * through the mapping table (a released entry is then ULA_ERANGE). la_host: n
 * addresses in host memory. Enqueued on `stream`, ordered after the group's
 * earlier calls like ula_append.
 * Validated on the host first: ULA_EINVAL (bad g or n < 0), ULA_ERANGE (address
 * outside [0, N) or not appended), ULA_EDUP (repeated), ULA_ESTATE; nothing
 * changes on error. */
int ula_release(ula_ctx* ctx, int32_t group, int32_t n, const int32_t* la_host, uint64_t stream);

/* One decode step (one scheduling round) of group g over n_sets x k selected
 * addresses (device memory, row-major, -1 = padding), section 3: de-duplicate
 * (first occurrence in row-major order) and look up once for the group; advance
 * the ring and fold the reused bucket into cold; move hits into the current
 * bucket; pick one victim per miss (free, cold, ring oldest -> newest, ascending
 * slot inside a bucket, never the current bucket); bring the missed rows in from
 * the host pool; then update the mapping table and owners and raise the
 * completion counter to the step number. Data path: the missed rows are read
 * into device memory in the same launch that marks the hits and plans the
 * victims; the victims' rows are staged in device memory as the missed rows
 * replace them; the staged rows reach the host slots their misses vacated
 * during the group's next step, beside that step's reads from the host (a miss
 * of a row evicted by the previous step reads its staged copy), or when
 * ula_read_rows or ula_release needs the host pool current. So the mapping
 * table can name a host slot for an evicted entry one step before its rows
 * land there; every GPU reader is unaffected (a row in the host pool is read
 * only by a later step of the group, which writes the staged rows first or
 * reads the staged copy). Enqueued on
 * `stream` with no host synchronisation.
 * Host errors: ULA_EINVAL (bad g, n_sets > max_sets, k > max_k, negative sizes),
 * ULA_ESTATE. Device errors (reported by ula_sync): ULA_ERANGE, ULA_ECAPACITY. */
int ula_step(ula_ctx* ctx, int32_t group, int32_t n_sets, int32_t k, const int32_t* sel_dev,
             uint64_t stream);

/* One decode step of group g with its appends (section 2: the new positions a
 * step produces are appended, then the step selects among all entries):
 * exactly ula_append(ctx, group, n_app, la_host, rows, rows_on_device, stream)
 * followed by ula_step(ctx, group, n_sets, k, sel_dev, stream), with the same
 * arguments, placement and results, in fewer launches: an append of at most 128
 * entries (256 under ULA_POLICY_LRU; and at most max_append) with rows in device
 * memory runs in the
 * step's first launch, beside the de-duplication, which does not read the
 * mapping table; other appends run as ula_append does, before the step.
 * n_app = 0 is a plain step. Both parts are validated on the host before
 * anything is enqueued: any host error of ula_append or ula_step is returned
 * with nothing changed. Device errors of the step are reported by ula_sync as
 * for ula_step; the appended entries stay appended. */
int ula_append_step(ula_ctx* ctx, int32_t group, int32_t n_app, const int32_t* la_host,
                    const void* rows, int32_t rows_on_device, int32_t n_sets, int32_t k,
                    const int32_t* sel_dev, uint64_t stream);

/* Gather layer `layer` of every selected entry of group g into out_dev
 * (device memory, n_sets x k x row_bytes bytes, packed; a -1 entry gives a zero
 * row). Reads the GPU pool through the mapping table after checking that the
 * group's completion counter equals the group's last step (section 3: readers
 * wait for the signal); call it once per layer of the group, or gather several
 * layers in one launch with ula_gather_layers. On a stream other
 * than the step's, order it after the step first (event, or a stream wait on
 * ula_flag_address reaching the step number): the counter check inside the
 * gather is a relaxed read that only catches a gather that runs before the
 * counter is raised (ULA_ENOTRESIDENT); the rows of an unordered gather that
 * finds the counter raised are undefined, since nothing orders its reads after
 * the step's writes on another cache. The group's later calls need no
 * ordering after the gather: the library makes the next launch that moves rows
 * out of GPU slots wait for it (see Threading). A gather that runs while the
 * group's next step fails on the device may find that step's error and write
 * nothing (ula_sync reports the error); a gather of an address appended only
 * after its step is an error, or undefined if that append runs beside it.
 * Host errors: ULA_EINVAL, ULA_ESTATE, ULA_ENOTRESIDENT (no step yet).
 * Device errors (reported by ula_sync): ULA_ENOTRESIDENT (counter not reached,
 * or an entry not on the GPU), ULA_ERANGE. */
int ula_gather(ula_ctx* ctx, int32_t group, int32_t layer, int32_t n_sets, int32_t k,
               const int32_t* sel_dev, void* out_dev, uint64_t stream);

/* Gather layers layer0 .. layer0 + n_layers - 1 of every selected entry of
 * group g in one launch (section 2: the layers of a group share one selection,
 * and the later layers are fetched while an earlier one is in use). out_dev
 * (device memory) holds n_layers per-layer buffers one after the other, each
 * n_sets x k x row_bytes bytes laid out as ula_gather writes it: the result is
 * exactly that of ula_gather(layer0 + i, out_dev + i * n_sets * k * row_bytes)
 * for each i. Since a slot keeps its layers side by side, each entry's layers
 * are read as one contiguous run. Same checks and errors as ula_gather, plus
 * ULA_EINVAL unless 0 <= layer0, 1 <= n_layers and layer0 + n_layers <=
 * layers_per_group. */
int ula_gather_layers(ula_ctx* ctx, int32_t group, int32_t layer0, int32_t n_layers, int32_t n_sets,
                      int32_t k, const int32_t* sel_dev, void* out_dev, uint64_t stream);

/* Wait for `stream`, then report the first latched device error of any group
 * (poisoning the context) or ULA_OK (section 3: a host waiter for the steps'
 * completion). per_group_out (nullable, num_groups entries) receives each
 * group's last step statistics (section 4: the GPU hit rate is hits over
 * distinct selected entries). Errors: ULA_EINVAL, ULA_EHIP, or the latched code. */
int ula_sync(ula_ctx* ctx, uint64_t stream, ula_step_stats* per_group_out);

/* Copy group g's canonical state (mapping table, owners, bucket bitsets, the
 * current bucket, the completion counter and the last step's statistics) into
 * caller host buffers, after synchronising the device. Staged evicted rows stay
 * staged: none of these fields depends on the host pool's bytes. Works on a
 * poisoned context. cur is derived from the counter (the ring advances once
 * per step, section 3), not read from the device. Errors: ULA_EINVAL (null
 * context or buffers, bad group), ULA_EHIP. */
int ula_export_state(ula_ctx* ctx, int32_t group, ula_state_host* out);

/* Read back the stored rows (all layers, layers_per_group x row_bytes bytes
 * each) of n appended entries of group g into host memory, from whichever pool
 * holds them (for checks of stored data; no passage of the pages behind it) (writes any staged evicted rows to the host pool and synchronises
 * the device first). ULA_ERANGE if an address was never
 * appended. */
int ula_read_rows(ula_ctx* ctx, int32_t group, int32_t n, const int32_t* la_host,
                  void* out_host);

/* Device address of group g's completion counter (int64, equals the last
 * completed step), for hipStreamWaitValue64 on another stream (section 3:
 * readers wait for the completion signal). A step that fails on the device
 * leaves the last completed step in the counter and sets bit 62, so a stream
 * waiting for the counter to be greater than or equal to that step's number is
 * released rather than left waiting; a gather it then issues is refused, and
 * ula_sync reports the failure. ula_export_state reports the counter without
 * that bit. */
int ula_flag_address(ula_ctx* ctx, int32_t group, void** dev_ptr);

/* Timing, off by default; ula_set_timing takes an OR of these flags (ULA_EINVAL
 * for unknown bits).
 *  - ULA_TIMING_STEP: events between the phases of every step. ula_read_timing
 *    gives, for the last step of group g, in milliseconds: [0] lookup +
 *    de-duplication, [1] hit marking + fold + victim selection, with the missed
 *    rows read in and the previous step's evicted rows written out over the
 *    host link in the same launch, [2] rows into the victim slots + commit +
 *    signal. It synchronises on the step's last event.
 *  - ULA_TIMING_GATHER: every gather launch records events in its own dispatch,
 *    so their interval is the kernel's execution alone (no launch overhead).
 *    ula_read_gather_timing synchronises on them and returns the summed kernel
 *    time and the number of launches since the last read (then resets both).
 *  - ULA_TIMING_LINK: the same for every step's host-link launch (the launch
 *    that reads the missed rows in and writes the previous step's evicted rows
 *    out while it marks hits and selects victims; under exact LRU, the first
 *    select pass, which carries that work); read by ula_read_link_timing.
 * Errors: ULA_EINVAL (unknown flag, null pointer, step timing never switched
 * on), ULA_EHIP. */
enum { ULA_TIMING_STEP = 1, ULA_TIMING_GATHER = 2, ULA_TIMING_LINK = 4 };
int ula_set_timing(ula_ctx* ctx, int32_t flags);
int ula_read_timing(ula_ctx* ctx, int32_t group, float* ms_out3);
int ula_read_gather_timing(ula_ctx* ctx, double* kernel_ms, int64_t* launches);
int ula_read_link_timing(ula_ctx* ctx, double* kernel_ms, int64_t* launches);

/* Release the context (not the caller's buffers). Waits for no stream.
 * Resource management only; no passage of the pages behind it. */
int ula_destroy(ula_ctx* ctx);

/* Text of an error code (also the last HIP error text for ULA_EHIP). Plumbing;
 * no passage of the pages behind it. */
const char* ula_strerror(int code);

/* Pinned, device-mapped host memory for the host pool (hipHostMalloc);
 * NULL on failure. ula_host_free returns ULA_OK or ULA_EHIP. Plumbing (section
 * 2's host pool lives in it). */
void* ula_host_alloc(size_t bytes);
int ula_host_free(void* p);

#ifdef __cplusplus
}
#endif

#endif /* ULA_H */
