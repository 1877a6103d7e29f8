/*
 * libkvx transfer state machine: the producer-side bookkeeping that decides
 * when each layer's KV write of a request is issued and when the request
 * counts as transferred.  The writes themselves are kvx_push_layer calls.
 *
 * It follows these passages of the pages:
 *   [PUSH] "Implementierungsdetails" steps 1-3: the consumer registers the
 *     block positions it reserved; registration and the producer's prefill
 *     may arrive in either order, and whichever is second starts the
 *     transfer; requests are matched by ID, including re-sent and retried
 *     ones.
 *   [MORI] §3.2: each layer's write is queued right after that layer's
 *     compute and runs after the layer's event; a write whose destination is
 *     not known yet is deferred and given up after a defer timeout; at the
 *     end of the forward pass the number of queued writes is sealed as the
 *     expected count and the request is done when that many writes finished.
 *   [MORI] §6: the outcome is judged over every layer batch (one failed layer
 *     fails the request even if later layers finished); a transfer timeout
 *     bounds a stuck write.
 *   [MORI] §3.1: the destination blocks of a failed request are reported so
 *     the consumer recomputes them.
 * (Page titles in kvx.h.)
 *
 * Readings where the pages leave a step open:
 *   - An attempt number orders re-sends of one request ID.  A message for an
 *     older attempt is ignored ("accepted" = 0).  A message for a newer
 *     attempt drops what was held for the older one.  Writes of the older
 *     attempt that were already enqueued still run; the caller must not
 *     reuse their destination blocks before they finish.
 *   - The recompute list of a FAILED or EXPIRED request is every destination
 *     block it registered.
 *   - A layer saved twice in one attempt counts once; saves after seal are
 *     not accepted.
 *   - The deferral clock starts at the first deferred write; the transfer
 *     clock at each layer's issue; a timeout fires once elapsed >= limit.
 *
 * Time is injected: every call that can start or expire work takes `now`
 * in seconds on a clock of the caller's choice.
 *
 * Threading: calls on one kvx_xfer are serialized internally (a mutex).
 * In device mode the calls build plans and record and query events: make
 * them while no graph capture is in progress in the process (a global-mode
 * capture on any stream would be invalidated).
 * Return values follow kvx.h (KVX_OK or KVX_E_*).  Unless a call lists
 * more: INVAL for a null handle or argument, HIP for a runtime failure
 * (device mode), NOMEM when host memory runs out.  `accepted` outputs
 * (nullable) report whether the message changed the state: 1 = applied,
 * 0 = ignored (stale attempt, finished request, duplicate).  Unlike other
 * outputs they are written whatever the return value: a registration
 * whose plan fails to build is applied (the request turns FAILED) and
 * returns the plan's error.
 *
 * Memory: a request's plan (and its device work list) is released when the
 * request finishes, once the writes already enqueued with it are done.  Its
 * record (state, layer states, recompute list) stays for queries until
 * kvx_xfer_forget.  The issued-write log is kept only with KVX_XFER_LOG.
 */
#ifndef KVX_XFER_H
#define KVX_XFER_H

#include "kvx.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Request states. */
enum { KVX_REQ_PENDING = 0, KVX_REQ_DONE = 1, KVX_REQ_FAILED = 2, KVX_REQ_EXPIRED = 3 };

/* kvx_xfer_config.flags */
#define KVX_XFER_HOST_ONLY 1u /* plans are host-only and nothing is launched; issued writes
                                 finish only through kvx_xfer_complete (CPU tests) */
#define KVX_XFER_LOG 2u       /* keep the log of issued writes that kvx_xfer_issued reads (tests,
                                 tracing); it grows with every write.  Without it nothing is
                                 logged, and memory is bounded by the requests held. */

typedef struct kvx_xfer_config {
  double defer_timeout_s;    /* pages' default: 60 */
  double transfer_timeout_s; /* pages' default: 30 */
  uint32_t flags;
} kvx_xfer_config;

typedef struct kvx_xfer_s kvx_xfer;

/* Create a state machine for writes out of `producer` on `stream` (the side
 * stream all writes and their completion events go to; NULL = null stream).
 * `cfg` NULL = the pages' defaults.  Errors: INVAL, NOMEM. */
int kvx_xfer_create(const kvx_pool* producer, const kvx_xfer_config* cfg, hipStream_t stream, kvx_xfer** out);

/* Wait for every write this object enqueued, then free it and its plans.
 * NULL is a no-op. */
void kvx_xfer_destroy(kvx_xfer* x);

/* Consumer registration ([PUSH] step 1): the consumer pool and the block IDs
 * it reserved for request `req` (n entries, copied).  The consumer pool must
 * outlive the request.  Starts any deferred writes if the producer side is
 * known.  Errors: INVAL; a plan error (RANGE, DUPDST, MISMATCH, ...) when the
 * transfer starts, after which the request is FAILED. */
int kvx_xfer_register(kvx_xfer* x, uint64_t req, uint32_t attempt, const kvx_pool* consumer,
                      const int32_t* dst_ids, int64_t n, double now, int32_t* accepted);

/* Producer side: tokens the request moves (kvx_tokens_to_move for P->D) and
 * its source block IDs (n entries, copied).  Same errors as register. */
int kvx_xfer_prefill(kvx_xfer* x, uint64_t req, uint32_t attempt, int64_t num_tokens, const int32_t* src_ids,
                     int64_t n, double now, int32_t* accepted);

/* Layer `layer` of the request has been computed; `ready` (nullable) fires
 * when its KV is in place.  The write is issued now if both sides are known,
 * else deferred (the dependency on `ready` is captured now, so the caller may
 * reuse the event).  Errors: INVAL, RANGE (layer), HIP. */
int kvx_xfer_save_layer(kvx_xfer* x, uint64_t req, uint32_t attempt, int32_t layer, hipEvent_t ready, double now,
                        int32_t* accepted);

/* kvx_xfer_save_layer for n requests at once, all gated by the same `ready`
 * (one save per layer for the whole batch, as an engine calls it after each
 * layer): the stream waits on `ready` once and the deferred writes share one
 * captured event.  accepted (nullable) receives n flags.  Equivalent to n
 * kvx_xfer_save_layer calls in order. */
int kvx_xfer_save_layer_many(kvx_xfer* x, int32_t layer, hipEvent_t ready, int64_t n, const uint64_t* reqs,
                             const uint32_t* attempts, double now, int32_t* accepted);

/* End of the forward pass: the writes queued so far are the expected ones. */
int kvx_xfer_seal(kvx_xfer* x, uint64_t req, uint32_t attempt, int32_t* accepted);

/* Observe finished writes (device mode) and apply the timeouts at `now`.
 * Completion is observed through one event recorded per poll behind the
 * writes issued since the previous poll, so a write is seen done at the
 * first poll after the one following its issue. */
int kvx_xfer_poll(kvx_xfer* x, double now);

/* Report the outcome of an issued write: ok = 0 marks it failed (a transport
 * error; device or host-only mode), ok = 1 marks it finished (host-only mode
 * only; KVX_E_INVAL otherwise). */
int kvx_xfer_complete(kvx_xfer* x, uint64_t req, uint32_t attempt, int32_t layer, int32_t ok);

/* Current attempt and state of a request; KVX_E_RANGE if unknown. */
int kvx_xfer_status(const kvx_xfer* x, uint64_t req, uint32_t* attempt, int32_t* state);

/* Requests that became DONE, FAILED or EXPIRED since the last call, in
 * increasing request ID; at most `cap` are reported (the rest stay for the
 * next call).  *n receives the number written. */
int kvx_xfer_pop_finished(kvx_xfer* x, uint64_t* reqs, uint32_t* attempts, int32_t* states, int64_t cap,
                          int64_t* n);

/* Destination blocks to recompute ([MORI] §3.1): all registered blocks of a
 * FAILED or EXPIRED request, none otherwise.  Same cap/n protocol as
 * kvx_plan_runs. */
int kvx_xfer_recompute_blocks(const kvx_xfer* x, uint64_t req, int32_t* out, int64_t cap, int64_t* n);

/* Issued writes in issue order, from index `first`: (request, attempt,
 * layer).  *n receives how many were written (at most cap).  Needs
 * KVX_XFER_LOG at creation; without it, KVX_E_INVAL. */
int kvx_xfer_issued(const kvx_xfer* x, int64_t first, uint64_t* reqs, uint32_t* attempts, int32_t* layers,
                    int64_t cap, int64_t* n);

/* Drop a finished request's record (its plan was released when it
 * finished).  KVX_E_INVAL if it is still PENDING, KVX_E_RANGE if unknown. */
int kvx_xfer_forget(kvx_xfer* x, uint64_t req);

#ifdef __cplusplus
}
#endif

#endif /* KVX_XFER_H */
