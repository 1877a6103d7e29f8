/*
 * libkvx -- paged-KV block transfer between a producer (prefill) pool and a
 * consumer (decode) pool on one MI355X (gfx950).
 *
 * Sources this ABI follows (cited by page title and section):
 *   [PUSH]  "Push-based KV transfer for vLLM prefill/decode disaggregation
 *           with NIXL" (AWS blog, German translation,
 *           www.spke.com/de/ai/article/3844)
 *   [MORI]  "vLLM MoRIIO KV Connector (single-node PD disaggregation)"
 *           (donggyun112.github.io knowledge-base note)
 *   [BIDIR] "Bidirectional KV-cache transfer for multi-turn workloads"
 *           (AWS blog, German translation, www.spke.com/de/ai/article/3845)
 *
 * Conventions shared by every call:
 *   - Return value: KVX_OK (0) or one of the KVX_E_* codes.  No call throws,
 *     aborts or prints.  kvx_last_error() holds a thread-local message for the
 *     last failing call on this thread.  Output parameters are written only
 *     when the call returns KVX_OK.  A null handle or a null required pointer
 *     is KVX_E_INVAL for every call that lists errors.
 *   - Ownership: the caller owns all pool memory, staging buffers, streams and
 *     events and must keep pool memory alive until enqueued work completes.
 *     The library owns the opaque kvx_pool / kvx_plan_t handles and each
 *     plan's device descriptor buffer.  Plans are immutable once built and
 *     may be used concurrently on several streams as long as the destination
 *     bytes of concurrent calls do not overlap.
 *   - Device calls are asynchronous: they enqueue on the given stream and
 *     return.  `ready` (may be NULL) is waited for with hipStreamWaitEvent
 *     before the kernel runs (skipped when it has already completed).
 *     Memory must be device memory of the current device.
 *   - Graph capture: device calls may be captured into a HIP graph.  Under
 *     capture, `ready` must have been recorded in the same capture (the wait
 *     becomes a graph edge), and the plan's descriptor upload must already
 *     have been observed complete on the host: call kvx_plan_wait before
 *     capturing (KVX_E_INVAL otherwise; the capture stays valid).
 *     kvx_plan must be called outside a capture (KVX_E_INVAL when its
 *     upload stream is capturing).  kvx_plan, kvx_plan_destroy_after and
 *     kvx_plan_reclaim allocate device memory or record and query events,
 *     which invalidates a capture in global mode on any stream: call them
 *     while no capture is in progress in the process.
 *   - Bytes are copied, never interpreted: bf16, fp8 or any other element type
 *     of 1, 2 or 4 bytes moves bit-exactly.
 */
#ifndef KVX_H
#define KVX_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVX_ABI_VERSION 7

/* Status codes. */
enum {
  KVX_OK = 0,
  KVX_E_INVAL = 1,       /* null pointer, negative count, short block list, bad flags */
  KVX_E_RANGE = 2,       /* block ID outside the pool, layer or head range out of bounds */
  KVX_E_DUPDST = 3,      /* a destination block is used twice within one plan */
  KVX_E_MISMATCH = 4,    /* the two pools' geometries are incompatible for the call */
  KVX_E_UNSUPPORTED = 5, /* alignment or a geometry limit: a base not 16-B aligned, row bytes not a
                            multiple of 16, block_size above 32768, a block of 2^31 B or more,
                            per-block scales with different block sizes per side */
  KVX_E_NOMEM = 6,       /* host or device allocation failed */
  KVX_E_HIP = 7          /* a HIP runtime or launch error; see kvx_last_error() */
};

/* Block layouts inside one (layer, K or V) region.  Each side maps block
 * positions onto its own physical layout ([PUSH] "Implementierungsdetails",
 * step 3). */
enum {
  KVX_NHD = 0, /* [block][slot][head][dim] */
  KVX_HND = 1  /* [block][head][slot][dim] */
};

/* kvx_plan flags. */
#define KVX_PLAN_HOST_ONLY 1u /* build the host tables only; no device upload,
                                 device calls on the plan return KVX_E_INVAL */
#define KVX_PLAN_OVERLAP 2u   /* the caller keeps several device calls of this
                                 plan in flight at once (e.g. layers alternating
                                 over two side streams): launches stream small
                                 pieces instead of filling the chip alone */
#define KVX_PLAN_RUNS 4u      /* a plan whose launches stream (see
                                 kvx_plan_launch_shape) and whose regions share
                                 one triple list keeps a run table instead of
                                 cut pieces: 16 bytes per triple (twice: in
                                 destination and in plan order) plus 4 bytes
                                 per 32 KiB; each workgroup finds the runs of
                                 its 4 KiB chunk itself.  Ignored for one-wave
                                 plans, state pools and regions or staging of
                                 4 GiB or more.  The copied bytes do not
                                 depend on it. */

/*
 * Pool descriptor: the paged KV cache of one layer group on one side, as
 * exchanged at the first handshake (KV base address, block size, per-layer
 * strides: [MORI] §3) and registered per layer ([MORI] §6,
 * register_kv_caches).  Layer l's K and V regions each hold num_blocks blocks
 * of block_size slots of num_heads rows of head_dim elements, in `layout`.
 * A block ID addresses the same block in every layer and in both K and V.
 *   k_base, v_base: host arrays of num_layers device pointers, 16-B aligned.
 *     Entries may repeat (several logical layers aliasing one slab).
 *     v_base NULL: each layer has one region only, the latent KV shared by
 *     keys and values of an MLA layer ([MORI] §6: layers of other shapes,
 *     MLA among them, get their own geometry); v_scale must be NULL then.
 *   k_scale, v_scale: NULL (no scales) or host arrays of num_layers device
 *     pointers to fp32[num_blocks], one scale per (layer, region, block),
 *     4-B aligned.  A scale travels with its block, unchanged.
 *   sliding_window: 0 for full attention; W > 0 for a sliding-window group
 *     whose queries see the last W positions, their own included ([MORI] §6).
 *     A transfer then skips the blocks the receiving side's next query no
 *     longer sees (see kvx_plan).
 * Requirements: all counts >= 1; elem_bytes in {1, 2, 4}; head_dim *
 * elem_bytes a multiple of 16, block_size <= 32768 and block_size *
 * num_heads * head_dim * elem_bytes < 2^31 (KVX_E_UNSUPPORTED otherwise);
 * sliding_window >= 0.  Zero-initialise the struct so that
 * fields added by later versions read as 0.
 * The library copies the descriptor; the arrays may be freed after the call.
 */
typedef struct kvx_pool_desc {
  int32_t num_layers, num_blocks, block_size, num_heads, head_dim;
  int32_t elem_bytes;
  int32_t layout;
  void* const* k_base;
  void* const* v_base;
  float* const* k_scale;
  float* const* v_scale;
  int32_t sliding_window;
} kvx_pool_desc;

/*
 * State-slot pool: the recurrent state of a mamba-like layer group ([MORI]
 * §6, hybrid models: the state is registered as two regions, the
 * convolution state and the SSM state, and moved slot by slot).  Region r of
 * layer l holds num_slots slots of slot_bytes[r] bytes; a slot ID addresses
 * the same slot in every layer and both regions.
 *   base[r]: host array of num_layers device pointers, 16-B aligned.
 * Requirements: counts >= 1; slot_bytes[r] >= 16 and a multiple of 16
 * (KVX_E_UNSUPPORTED otherwise).
 */
typedef struct kvx_state_pool_desc {
  int32_t num_layers, num_slots;
  int64_t slot_bytes[2];
  void* const* base[2];
} kvx_state_pool_desc;

typedef struct kvx_pool kvx_pool;
typedef struct kvx_plan_s kvx_plan_t;

/* One merged run: blocks src0..src0+nblk-1 -> dst0..dst0+nblk-1, the last
 * block holding `tail` tokens (block_size unless it ends its request). */
typedef struct kvx_run {
  int32_t src0, dst0, nblk, tail;
} kvx_run;

/* One contiguous copy inside a (layer, K/V) region: byte offsets relative to
 * the region's base pointer on each side. */
typedef struct kvx_triple {
  int64_t src_off, dst_off, len;
} kvx_triple;

/* ABI version (KVX_ABI_VERSION of the built library). */
int32_t kvx_abi_version(void);

/* Static name of a status code; never NULL. */
const char* kvx_status_str(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* kvx_last_error(void);

/* Tokens a consumer takes from the producer: prompt_len - num_computed - 1,
 * clamped at 0.  The consumer always recomputes the final prompt token
 * ([MORI] §3.1, READ mode scheduler).  Callers pass the result to kvx_plan;
 * D->P reuse passes the reusable prefix itself (no -1). */
int64_t kvx_tokens_to_move(int64_t prompt_len, int64_t num_computed);

/* 1 if a reusable prefix of `reusable_tokens` should be pulled rather than
 * recomputed, i.e. reusable_tokens >= threshold; else 0.  The pages' default
 * threshold is 64 tokens ([BIDIR] "KV-Recompute-Schwellenwert"). */
int32_t kvx_should_reuse(int64_t reusable_tokens, int64_t threshold);

/* Register one side's KV cache.  Host-only: no device call is made.
 * Errors: INVAL (null/invalid field), UNSUPPORTED (a base not 16-byte or a
 * scale array not 4-byte aligned, head_dim*elem_bytes not a multiple of 16,
 * block_size above 32768, a block of 2^31 bytes or more per region), NOMEM. */
int kvx_pool_create(const kvx_pool_desc* desc, kvx_pool** out);

/* Register a state-slot pool.  Host-only.  Errors: INVAL, UNSUPPORTED, NOMEM. */
int kvx_state_pool_create(const kvx_state_pool_desc* desc, kvx_pool** out);

/* Free a pool handle (never the pool memory).  NULL is a no-op.  Plans built
 * from the pool stay valid: they hold their own copy of the descriptors. */
void kvx_pool_destroy(kvx_pool* pool);

/*
 * Build a transfer plan from `src` to `dst` for `num_requests` requests.
 *   num_tokens[r]: tokens request r moves (>= 0); the caller applies the
 *     final-token rule (kvx_tokens_to_move) for P->D.
 *   src_offsets[r], src_offsets[r+1] (and dst_offsets likewise): CSR bounds
 *     of request r's block list in src_ids (dst_ids); non-decreasing, first
 *     entry >= 0.  Only the first ceil(num_tokens[r] / block_size) entries of
 *     each list are used, block_size being that side's; later entries are
 *     ignored and not validated.
 *   src_ids / dst_ids: block IDs of the producer / consumer pool.
 * Token t of a request sits in source block src_ids[t / BS_src], slot
 * t % BS_src, and lands in destination block dst_ids[t / BS_dst], slot
 * t % BS_dst: each side maps block positions onto its own layout, so block
 * sizes may differ ([PUSH] "Implementierungsdetails" step 3).  With equal
 * block sizes the block pairs of each request are merged, in list order,
 * into maximal runs consecutive on both sides; runs never cross requests.
 * This is the merge of contiguous blocks into larger transfer regions done by
 * the push connector's background thread ([PUSH] "Threading-Modell") and by
 * the per-layer offset computation ([MORI] §3.1, §6).  When both pools have
 * the same head count and layout the plan also holds the per-region triple
 * list and the device work list for kvx_push_layer / kvx_pack / kvx_unpack;
 * otherwise only kvx_copy_heads may use it.
 * Sliding-window pools: request r's next query, at position n =
 * num_tokens[r], sees positions n-W+1 .. n.  Blocks holding none of them
 * are skipped: the move covers tokens [t0, n), t0 being the later of the two
 * sides' starts of the block that holds position max(0, n-W+1).  List
 * entries of skipped blocks are neither read nor validated (an engine's null
 * block may stand there).
 * State-slot pools (both sides): a request with num_tokens[r] >= 1 moves its
 * slot, the first entry of its list on each side, in both regions; one with
 * 0 tokens moves nothing.  Each moving request is one run (tail 1), and each
 * region's triples merge neighbouring slots.
 * Pools must be of the same kind (KVX_E_MISMATCH otherwise).  Attention pools
 * must agree on num_layers, head_dim, elem_bytes, region count, scale
 * presence and sliding_window (KVX_E_MISMATCH otherwise); pools with scales
 * must also agree on block_size (KVX_E_UNSUPPORTED: a per-block scale has no
 * single source block otherwise).  State pools must agree on num_layers and
 * slot_bytes (KVX_E_MISMATCH).  src == dst is KVX_E_INVAL.
 * Unless KVX_PLAN_HOST_ONLY is set the device work list is uploaded on
 * `upload_stream` (NULL = the null stream); later device calls on any stream
 * are ordered after the upload.  The plan owns that one device buffer,
 * carved from the library's work-list arena on the current device: 32 B per
 * piece of at most 32 KiB (twice for a plan in a one-wave launch shape,
 * whose batched launches read a destination-ordered copy) plus 16 B per
 * planned block.  The arena takes chunks of at least 64 MiB from hipMalloc
 * and keeps them for reuse until the process ends (hipFree would
 * synchronize the whole device); it holds the peak of live work lists.
 * Validation order per request: token count, list lengths, source IDs, then
 * destination IDs.  Errors: INVAL (also: upload_stream is capturing a
 * graph), RANGE (ID outside its pool), DUPDST (a dst ID used twice in the
 * plan), MISMATCH, UNSUPPORTED, NOMEM, HIP.
 */
int kvx_plan(const kvx_pool* src, const kvx_pool* dst, int32_t num_requests,
             const int64_t* num_tokens, const int64_t* src_offsets, const int64_t* dst_offsets,
             const int32_t* src_ids, const int32_t* dst_ids, uint32_t flags,
             hipStream_t upload_stream, kvx_plan_t** out);

/*
 * kvx_plan without any device allocation, for callers that cannot allocate
 * device memory (code that runs while a stream is being captured elsewhere
 * in the process, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, result and errors as kvx_plan, except that the plan's
 * device work list goes into a static scratch array of 16 MiB that the
 * library holds on each device it runs on, until the process ends, and that
 * the upload is waited for on the host before the call returns (no event is
 * created).  Nothing else is allocated on the device, and no hipMalloc,
 * hipFree or other allocating runtime call is made; the host tables use the
 * C++ heap as kvx_plan's do.
 * The array is shared by every call on the device and keeps only the last
 * call's work list: a plan built this way is valid until the next
 * kvx_plan_noalloc on the same device, after which its device calls return
 * KVX_E_INVAL.  Building a plan while device calls of the previous one are
 * still running on the device races with them, as do concurrent calls.
 * Destroying such a plan frees no device memory (and waits for nothing).
 * Errors: those of kvx_plan; INVAL also for KVX_PLAN_HOST_ONLY; NOMEM when
 * the work list exceeds the array (KVX_PLAN_RUNS keeps streaming work
 * lists small). */
int kvx_plan_noalloc(const kvx_pool* src, const kvx_pool* dst, int32_t num_requests,
                     const int64_t* num_tokens, const int64_t* src_offsets, const int64_t* dst_offsets,
                     const int32_t* src_ids, const int32_t* dst_ids, uint32_t flags,
                     hipStream_t upload_stream, kvx_plan_t** out);

/* Copy the run table into out[0..cap); *n receives the run count.  With
 * out == NULL or cap < count only *n is written (and KVX_OK returned).
 * Runs are block pairs, defined for equal block sizes only (KVX_E_MISMATCH
 * otherwise; the triples describe such plans).  A state plan has one run per
 * moving request: its slot pair, nblk 1, tail 1. */
int kvx_plan_runs(const kvx_plan_t* plan, kvx_run* out, int64_t cap, int64_t* n);

/* The (src_off, dst_off, len) list of one (layer, region) pair (kv: 0 = K,
 * 1 = V; the latent region of an MLA pool is 0; a state pool's regions are 0
 * = conv, 1 = SSM): maximal contiguous byte ranges in plan order, the list
 * handed to one batch transfer per layer ([MORI] §6).  Offsets are relative
 * to that layer's region base on each side; the list is the same for every
 * layer, and for K and V.  NHD gives one triple per run; HND gives the run's
 * full blocks plus one range per head of a partly filled last block.
 * Same cap/n protocol as kvx_plan_runs.  Errors: RANGE, MISMATCH (no
 * triples: different head count or layout). */
int kvx_plan_triples(const kvx_plan_t* plan, int32_t layer, int32_t kv,
                     kvx_triple* out, int64_t cap, int64_t* n);

/* Launch shape of a plan's copy kernels, chosen when the plan is built from
 * its own triples: every workgroup of kvx_push_layer / kvx_pack /
 * kvx_unpack has `lanes` lanes, each keeping `vectors` 16-byte vectors in
 * flight, and copies one piece of at most piece_bytes; `pieces` is the
 * number of such workgroups in one layer's launch (all regions, scale
 * workgroups not counted).  For diagnostics and tuning only:
 * the copied bytes do not depend on it. */
typedef struct kvx_launch_shape {
  int64_t pieces;
  int32_t piece_bytes, lanes, vectors;
  int32_t run_table; /* 1: the plan keeps run tables (KVX_PLAN_RUNS honoured): `pieces`
                        counts 4 KiB chunks of its flat space, found in the kernel */
} kvx_launch_shape;

/* Errors: INVAL (null), MISMATCH (no push work list). */
int kvx_plan_launch_shape(const kvx_plan_t* plan, kvx_launch_shape* out);

/* Wait on the host until the plan's descriptor upload has completed, so
 * that its device calls can be captured into a graph.  Call it outside a
 * capture.  A host-only plan, or one already observed, returns at once.
 * Errors: INVAL (null plan), HIP. */
int kvx_plan_wait(const kvx_plan_t* plan);

/* Bytes one layer's push reads and writes (every region's payload plus
 * scales), into *read_bytes and *write_bytes.  Errors: INVAL (null),
 * MISMATCH (pools differ in head count or layout: no push). */
int kvx_plan_bytes(const kvx_plan_t* plan, int64_t* read_bytes, int64_t* write_bytes);

/* Free a plan.  Device calls already enqueued with it may still be running
 * on any stream, so this first waits until the device is idle
 * (hipDeviceSynchronize).  NULL is a no-op. */
void kvx_plan_destroy(kvx_plan_t* plan);

/* Free a plan without waiting on the host: it is freed once the work
 * enqueued on `stream` so far has finished.  The caller guarantees that no
 * other stream still has work with the plan in flight (or that `stream`
 * already waits for it), and enqueues nothing more with it.  The memory is
 * reclaimed by a later kvx_plan (device plans), kvx_plan_destroy_after or
 * kvx_plan_reclaim call after that point.  A host-only plan is freed at
 * once; NULL is a no-op.  Errors: INVAL (`stream` is capturing a graph),
 * NOMEM, HIP. */
int kvx_plan_destroy_after(kvx_plan_t* plan, hipStream_t stream);

/* Free the plans released with kvx_plan_destroy_after whose work has
 * finished; with wait != 0, wait for the rest first.  *pending (nullable)
 * receives how many remain.  Errors: HIP. */
int kvx_plan_reclaim(int32_t wait, int64_t* pending);

/*
 * Layerwise push: copy layer `layer`'s bytes of every planned token in every
 * region (and the scales of every planned block; for state pools, every
 * planned slot) from the src pool into the dst pool, after `ready` fires, on
 * `stream`.  This is the per-layer write that
 * starts once that layer's compute is done and overlaps the next layer's
 * compute ([MORI] §3.2, save_kv_layer and the event sync before the write;
 * [PUSH] "Implementierungsdetails" step 3).  Slots past a request's last
 * token keep their old bytes, so the consumer never receives the final
 * prompt token ([MORI] §3.1).
 * Errors: INVAL (host-only plan, null plan), RANGE (layer), MISMATCH (pools
 * differ in head count or layout), HIP.
 */
int kvx_push_layer(const kvx_plan_t* plan, int32_t layer, hipEvent_t ready, hipStream_t stream);

/* kvx_push_layer whose kernel records its own start and end timestamps into
 * `started` / `finished` (events created with timing enabled; either may be
 * NULL).  The timestamps are taken from the kernel dispatch itself, so no
 * extra queue packets are added: hipEventElapsedTime(started, finished) is
 * the kernel's execution time.  A plan whose work list is empty launches
 * nothing and leaves both events untouched.  Same errors as kvx_push_layer. */
int kvx_push_layer_timed(const kvx_plan_t* plan, int32_t layer, hipEvent_t ready, hipStream_t stream,
                         hipEvent_t started, hipEvent_t finished);

/*
 * Several layer pushes with one kernel launch: pair i copies layer layers[i]
 * of plans[i] exactly as kvx_push_layer would, all after `ready` fires, on
 * `stream`.  Unlike n kvx_push_layer calls, the pairs' copies may run at the
 * same time, so no two pairs may write the same destination bytes (sources
 * may overlap).  This is one batch write per layer over many requests'
 * (offset, offset, size) lists ([MORI] §6), for requests whose plans were
 * built at different times (a transfer starts when its consumer registers),
 * and the flush of several deferred layers of one request.  Plans may have
 * different pools.  Pairs with the same region count share launches of up
 * to 32 entries, in their order (one-region and two-region pairs gather
 * apart, so the launches of the two kinds may go out in either order); the
 * per-block scales of a launch's pairs follow in one small launch behind
 * it; pairs whose work list alone fills a launch, and run-table plans, run
 * as launches of their own, in order.  A
 * shared launch runs in its plans' common one-wave shape when it stays
 * within about one round of it, else as 4 KiB chunks of every plan's pieces,
 * each plan's taken in destination order (see kvx_plan_launch_shape).
 * Everything is ordered after `ready`
 * and before later work on `stream`.  All pairs are validated before
 * anything is enqueued.
 * Errors: INVAL (n < 0, null arrays with n > 0, a null or host-only plan),
 * RANGE (a layer), MISMATCH (a plan without a push work list), HIP.
 */
int kvx_push_many(const kvx_plan_t* const* plans, const int32_t* layers, int32_t n, hipEvent_t ready,
                  hipStream_t stream);

/* kvx_push_many whose first kernel records its start timestamp into
 * `started` and whose last kernel records its end into `finished` (events
 * with timing enabled; either may be NULL), taken from the dispatches
 * themselves as in kvx_push_layer_timed: the elapsed time between them spans
 * the call's launches.  Nothing launched leaves both untouched.  Same errors
 * as kvx_push_many. */
int kvx_push_many_timed(const kvx_plan_t* const* plans, const int32_t* layers, int32_t n, hipEvent_t ready,
                        hipStream_t stream, hipEvent_t started, hipEvent_t finished);

/*
 * Layer write queue of one stream.  In push mode the producer queues each
 * layer's write right after that layer's compute; the write goes out once
 * the layer's event has fired, and at the end of the forward pass the
 * producer waits for all of them ([MORI] §3.2, WRITE mode, with the event
 * sync before each layer write; [MORI] §6, the worker hooks save_kv_layer
 * and wait_for_save).  kvx_queue_push is the save of one layer,
 * kvx_queue_flush the point after which work enqueued on the stream (an
 * event for wait_for_save) follows every queued write.
 * Each launch on a stream costs a few microseconds beyond its copy, which a
 * layer of tens of megabytes feels.  The queue therefore keeps at most two
 * launch groups of its writes in flight on its stream: a write that is ready
 * (its event has fired, or is NULL) while two groups still run waits in the
 * queue, and the ready writes at its front leave together, as one launch
 * group (kvx_push_many's batched launches for pushes, kvx_copy_heads_layers'
 * for head-slice writes), as soon as a group finishes.  A write whose event
 * has not fired blocks the writes queued behind it until it fires (writes
 * leave in queue order).  No write starts before its own event has fired;
 * writes of one group may run at the same time, so writes queued between
 * two flushes must not write the same destination bytes (repeating an
 * identical write is harmless).  The queue observes its launches and the
 * ready events only through event queries, so it never blocks the host.
 * `ready` is consumed at the push, as a stream wait would: the write waits
 * for the event's recording at that moment, and the caller may re-record or
 * destroy the event right after.  (An event not yet fired is mirrored by an
 * event of the queue's own, recorded behind a wait on a helper stream that
 * the queue creates at the default priority and that carries no kernels.)
 * A queue belongs to one stream on the current device and is not for graph
 * capture (KVX_E_INVAL while the stream captures).  Plans must stay alive
 * until the flush that enqueues their writes, then as for kvx_push_layer.
 */
typedef struct kvx_queue kvx_queue;

/* Create the write queue of `stream` (NULL = the null stream).
 * Errors: INVAL (null out, stream capturing), NOMEM, HIP. */
int kvx_queue_create(hipStream_t stream, kvx_queue** out);

/* Queue the write of layer `layer` of `plan` (what kvx_push_layer would
 * copy), to go out after `ready` (nullable) fires.  May enqueue launches of
 * earlier writes.  On an error the writes still queued are dropped.
 * Errors: INVAL (null queue or plan, host-only plan, stream capturing),
 * RANGE (layer), MISMATCH (a plan without a push work list), HIP. */
int kvx_queue_push(kvx_queue* q, const kvx_plan_t* plan, int32_t layer, hipEvent_t ready);

/* Queue one TP rank's head-slice write of layer `layer` of `plan` (what
 * kvx_copy_heads would copy: source heads [src_head0, src_head0 +
 * num_heads) onto destination heads [dst_head0, ...), each side in its own
 * layout, scales with their blocks), to go out after `ready` (nullable)
 * fires: the layerwise write that addresses each target TP rank ([PUSH]
 * "Implementierungsdetails" step 3; [MORI] §3.2 for the per-layer trigger).
 * Ready head-slice writes of one plan and slice that leave together share
 * launches of up to 32 layers, as in kvx_copy_heads_layers; a group's pushes
 * go out before its head-slice writes.  Errors: those of kvx_copy_heads for
 * one layer, INVAL for a null queue or a capturing stream; on an error the
 * writes still queued are dropped. */
int kvx_queue_push_heads(kvx_queue* q, const kvx_plan_t* plan, int32_t layer, int32_t src_head0,
                         int32_t dst_head0, int32_t num_heads, hipEvent_t ready);

/* Enqueue every queued write on the queue's stream, each still waiting for
 * its own event (a stream wait for an event not yet observed fired), so that
 * work enqueued on the stream afterwards follows them all.  Returns without
 * waiting on the host.  Errors: INVAL (null queue, stream capturing), HIP
 * (the writes still queued are dropped). */
int kvx_queue_flush(kvx_queue* q);

/* Writes queued so far, launch groups enqueued so far (each group is one
 * kvx_push_many launch sequence) and the kernel launches of those groups
 * (`launches` may be NULL).  Errors: INVAL (null q, writes or groups). */
int kvx_queue_stats(const kvx_queue* q, int64_t* writes, int64_t* groups, int64_t* launches);

/* Flush, then free the queue.  NULL is a no-op (KVX_OK).  Returns the
 * flush's status; the queue is freed in every case. */
int kvx_queue_destroy(kvx_queue* q);

/* Staging bytes for layers [l0, l1): (l1 - l0) * sum over the layer's
 * regions of (payload + scale segment), where payload = sum of the region's
 * triple lengths and the scale segment is 4 bytes per planned block rounded
 * up to 16 (0 without scales).
 * Errors: INVAL (null), RANGE (0 <= l0 <= l1 <= num_layers violated),
 * MISMATCH (pools differ in head count or layout). */
int kvx_staging_bytes(const kvx_plan_t* plan, int32_t l0, int32_t l1, int64_t* bytes);

/*
 * Gather layers [l0, l1) of the planned bytes from the src pool into a
 * contiguous staging buffer (what a NIC would read), laid out for each layer
 * in order, region by region (K then V; conv then SSM): the region's
 * triples' source bytes in plan order, then
 * (with scales) the planned blocks' fp32 scales in plan order, zero-padded to
 * 16 bytes.  `staging` is device memory, 16-B aligned, of `cap` bytes >=
 * kvx_staging_bytes.  The src pool of the plan is read; nothing else is
 * written.  Launches: a plan of cut pieces copies up to 32 layers per
 * kernel launch (fewer when a launch would exceed 2^22 workgroups of 4 KiB),
 * with the scales, if any, in one small launch behind each; a run-table
 * plan one layer per launch.  Errors: INVAL (null, cap too
 * small, host-only plan), RANGE, MISMATCH, UNSUPPORTED (staging
 * misaligned), HIP.
 */
int kvx_pack(const kvx_plan_t* plan, int32_t l0, int32_t l1, void* staging, int64_t cap,
             hipStream_t stream);

/* Scatter a staging buffer laid out as by kvx_pack into the plan's dst pool.
 * kvx_unpack(kvx_pack(x)) leaves dst exactly as kvx_push_layer over the same
 * layers would.  Same errors as kvx_pack. */
int kvx_unpack(const kvx_plan_t* plan, int32_t l0, int32_t l1, const void* staging, int64_t cap,
               hipStream_t stream);

/*
 * Layout and head-slice transform for one layer: for every planned token,
 * source heads [src_head0, src_head0 + num_heads) land on destination heads
 * [dst_head0, dst_head0 + num_heads), each side addressed in its own layout
 * and head count (NHD <-> HND); planned blocks' scales travel unchanged.
 * This is one TP rank's share of a write that addresses each target TP rank
 * ([PUSH] "Implementierungsdetails" step 3; rank mapping in [MORI] §6).
 * num_heads == 0 is a no-op (the ready wait is still enqueued).
 * Errors: INVAL (negative head index/count, host-only plan), RANGE (layer or
 * head slice outside either pool), MISMATCH (state pools have no heads), HIP.
 */
int kvx_copy_heads(const kvx_plan_t* plan, int32_t layer, int32_t src_head0, int32_t dst_head0,
                   int32_t num_heads, hipEvent_t ready, hipStream_t stream);

/*
 * kvx_copy_heads for every layer in [l0, l1), the same head slice in each:
 * a TP rank's share of several layers whose KV is complete, as when a
 * request's layers are written out together.  Up to 32 layers share one
 * kernel launch (one launch per layer when a layer's planned blocks alone
 * fill half a launch's 2^22 workgroups).  Everything is ordered after
 * `ready`.  Errors: those of kvx_copy_heads, with RANGE for a layer range
 * outside [0, num_layers] or l1 < l0; an empty range is a no-op.
 */
int kvx_copy_heads_layers(const kvx_plan_t* plan, int32_t l0, int32_t l1, int32_t src_head0, int32_t dst_head0,
                          int32_t num_heads, hipEvent_t ready, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVX_H */
