// Layer write queue of one stream (kvx_queue_* in kvx.h).
//
// In push mode the producer queues each layer's write right after that
// layer's compute, and the write goes out once the layer's event has fired;
// at the end of the forward pass it waits for all of them ([MORI] §3.2,
// WRITE mode; the worker hooks save_kv_layer and wait_for_save, [MORI] §6).
// On a GPU every write is a kernel launch, and back-to-back launches on one
// queue cost a few microseconds each on top of the copy.  The queue keeps at
// most kInflight launch groups in flight on its stream; writes that become
// ready while those run are held and leave together in the next launch
// group (kvx_push_many's batched launch), so the fixed cost is paid per
// group instead of per layer when writes back up, and every write still
// starts only after its own layer's event.  A write may also be one TP
// rank's head slice of a layer (kvx_copy_heads), for a consumer whose ranks
// each hold a share of the heads ([PUSH] "Implementierungsdetails" step 3);
// such writes batch like kvx_copy_heads_layers.

#include <hip/hip_runtime.h>

#include <deque>
#include <mutex>
#include <vector>

#include "kvx_internal.h"

namespace {

constexpr int kInflight = 2;

struct Entry {
  const kvx_plan_t* plan;
  int32_t layer;
  hipEvent_t ready;  // the queue's own copy of the caller's event; NULL once observed fired
  bool heads;        // a head-slice write (the slice below) rather than a push
  int32_t src_head0, dst_head0, num_heads;
};

}  // namespace

struct kvx_queue {
  hipStream_t stream = nullptr;
  // Helper stream that turns a caller's event into one of the queue's own:
  // a wait for the caller's event, then a record of an owned event.  The
  // caller's event is consumed at the push (as by a stream wait) and may be
  // re-recorded or destroyed right after.  It carries no kernels.
  hipStream_t aux = nullptr;
  std::vector<hipEvent_t> free_events;
  std::vector<hipEvent_t> all_events;
  std::mutex mu;
  std::deque<Entry> pending;
  hipEvent_t done[kInflight] = {};  // recorded behind each launch group, a ring, oldest at `head`
  int head = 0, busy = 0;
  int64_t writes = 0, groups = 0, launches = 0;
};

namespace kvx {
namespace {

void release_event(kvx_queue* q, hipEvent_t e) {
  if (e) q->free_events.push_back(e);
}

// An owned event that fires when `ready` (as recorded now) has fired.
int mirror_event(kvx_queue* q, hipEvent_t ready, hipEvent_t* out) {
  hipEvent_t e;
  if (!q->free_events.empty()) {
    e = q->free_events.back();
    q->free_events.pop_back();
  } else {
    const hipError_t c = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (c != hipSuccess) return fail_hip(c, "kvx_queue: hipEventCreateWithFlags");
    q->all_events.push_back(e);
  }
  hipError_t r = hipStreamWaitEvent(q->aux, ready, 0);
  if (r == hipSuccess) r = hipEventRecord(e, q->aux);
  if (r != hipSuccess) {
    q->free_events.push_back(e);
    return fail_hip(r, "kvx_queue: mirroring the ready event");
  }
  *out = e;
  return KVX_OK;
}

// 1: the entry may go out now (no event, or its event has fired); 0: not
// yet; negative: -status of a failed query.
int entry_ready(kvx_queue* qu, Entry& e) {
  if (!e.ready) return 1;
  const hipError_t q = hipEventQuery(e.ready);
  if (q == hipSuccess) {
    release_event(qu, e.ready);
    e.ready = nullptr;
    return 1;
  }
  if (q == hipErrorNotReady) return 0;
  return -fail_hip(q, "kvx_queue: hipEventQuery(ready)");
}

int retire(kvx_queue* q) {
  while (q->busy > 0) {
    const hipError_t e = hipEventQuery(q->done[q->head]);
    if (e == hipErrorNotReady) break;
    if (e != hipSuccess) return fail_hip(e, "kvx_queue: hipEventQuery(launch)");
    q->head = (q->head + 1) % kInflight;
    --q->busy;
  }
  return KVX_OK;
}

// The event that will mark the end of the next launch group.  When the ring
// is full its oldest group is dropped from tracking (stream order: it
// finishes before the next one).
hipEvent_t next_done(kvx_queue* q) {
  if (q->busy == kInflight) {
    q->head = (q->head + 1) % kInflight;
    --q->busy;
  }
  return q->done[(q->head + q->busy) % kInflight];
}

// Enqueue a group's launches: its pushes, then its head-slice writes.  With
// `done`, the group's last kernel records its end into it from its own
// dispatch (no marker packet behind it); a group that launched nothing
// records it on the stream instead.
int launch(kvx_queue* q, const std::vector<Entry>& group, hipEvent_t done) {
  const int64_t before = q->launches;
  std::vector<const kvx_plan_t*> plans;
  std::vector<int32_t> layers;
  std::vector<HeadsWrite> heads;
  for (const Entry& e : group) {
    if (e.heads) {
      heads.push_back(HeadsWrite{e.plan, e.layer, e.src_head0, e.dst_head0, e.num_heads});
    } else {
      plans.push_back(e.plan);
      layers.push_back(e.layer);
    }
  }
  if (!plans.empty()) {
    const int rc = push_batch(plans.data(), layers.data(), int32_t(plans.size()), q->stream, nullptr, done,
                              &q->launches);
    if (rc) return rc;
  }
  if (!heads.empty()) {
    const int rc = heads_batch(heads.data(), int32_t(heads.size()), q->stream, done, &q->launches);
    if (rc) return rc;
  }
  if (done) {
    if (q->launches == before) {
      const hipError_t e = hipEventRecord(done, q->stream);
      if (e != hipSuccess) return fail_hip(e, "kvx_queue: hipEventRecord");
    }
    ++q->busy;
    ++q->groups;
  }
  return KVX_OK;
}

void drop_pending(kvx_queue* q) {
  for (Entry& e : q->pending) release_event(q, e.ready);
  q->pending.clear();
}

// Launch the ready front of the queue while fewer than kInflight groups run.
int pump(kvx_queue* q) {
  int rc = retire(q);
  if (rc) return rc;
  std::vector<Entry> group;
  while (q->busy < kInflight && !q->pending.empty()) {
    size_t n = 0;
    while (n < q->pending.size()) {
      const int r = entry_ready(q, q->pending[n]);
      if (r < 0) return -r;
      if (r == 0) break;
      ++n;
    }
    if (n == 0) break;
    group.assign(q->pending.begin(), q->pending.begin() + std::ptrdiff_t(n));
    q->pending.erase(q->pending.begin(), q->pending.begin() + std::ptrdiff_t(n));
    rc = launch(q, group, next_done(q));
    if (rc) return rc;
  }
  return KVX_OK;
}

// Enqueue every queued write: ready ones merged, each one still waiting for
// its event behind a stream wait for that event.
int flush(kvx_queue* q) {
  int rc = pump(q);
  if (rc) return rc;
  if (q->pending.empty()) return KVX_OK;
  std::vector<Entry> group;
  std::deque<Entry> todo;
  todo.swap(q->pending);
  for (Entry& e : todo) {
    const int r = entry_ready(q, e);
    if (r < 0) return -r;
    if (r == 0) {
      rc = launch(q, group, nullptr);
      if (rc) return rc;
      group.clear();
      rc = wait_event(e.ready, q->stream);
      release_event(q, e.ready);   // the wait has taken the event's state
      e.ready = nullptr;
      if (rc) return rc;
    }
    group.push_back(e);
  }
  return launch(q, group, next_done(q));
}

}  // namespace
}  // namespace kvx

using namespace kvx;

extern "C" {

int kvx_queue_create(hipStream_t stream, kvx_queue** out) {
  if (!out) return fail(KVX_E_INVAL, "kvx_queue_create: null out");
  if (stream_capturing(stream)) return fail(KVX_E_INVAL, "kvx_queue_create: the stream is capturing a graph");
  kvx_queue* q = new (std::nothrow) kvx_queue;
  if (!q) return fail(KVX_E_NOMEM, "kvx_queue_create: out of host memory");
  q->stream = stream;
  hipError_t e = hipStreamCreateWithFlags(&q->aux, hipStreamNonBlocking);
  if (e != hipSuccess) {
    delete q;
    return fail_hip(e, "kvx_queue_create: hipStreamCreateWithFlags");
  }
  for (int i = 0; i < kInflight; ++i) {
    e = hipEventCreate(&q->done[i]);   // timing enabled: a kernel dispatch records into it
    if (e != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(q->done[j]);
      (void)hipStreamDestroy(q->aux);
      delete q;
      return fail_hip(e, "kvx_queue_create: hipEventCreate");
    }
  }
  *out = q;
  return KVX_OK;
}

// Queue an already validated write behind `ready` (nullable).
static int queue_write(kvx_queue* q, Entry en, hipEvent_t ready, const char* fn) {
  std::lock_guard<std::mutex> lk(q->mu);
  if (stream_capturing(q->stream)) return fail(KVX_E_INVAL, "%s: the stream is capturing a graph", fn);
  if (ready) {
    const hipError_t r = hipEventQuery(ready);
    if (r == hipErrorNotReady) {
      const int rc = mirror_event(q, ready, &en.ready);
      if (rc) return rc;
    } else if (r != hipSuccess) {
      return fail_hip(r, "kvx_queue: hipEventQuery(ready)");
    }
  }
  q->pending.push_back(en);
  ++q->writes;
  const int rc = pump(q);
  if (rc) drop_pending(q);
  return rc;
}

int kvx_queue_push(kvx_queue* q, const kvx_plan_t* plan, int32_t layer, hipEvent_t ready) {
  if (!q) return fail(KVX_E_INVAL, "kvx_queue_push: null queue");
  const int rc = check_push_pair(plan, layer, "kvx_queue_push", 0);
  if (rc) return rc;
  return queue_write(q, Entry{plan, layer, nullptr, false, 0, 0, 0}, ready, "kvx_queue_push");
}

int kvx_queue_push_heads(kvx_queue* q, const kvx_plan_t* plan, int32_t layer, int32_t src_head0,
                         int32_t dst_head0, int32_t num_heads, hipEvent_t ready) {
  if (!q) return fail(KVX_E_INVAL, "kvx_queue_push_heads: null queue");
  const int rc = check_heads_write(HeadsWrite{plan, layer, src_head0, dst_head0, num_heads}, "kvx_queue_push_heads");
  if (rc) return rc;
  return queue_write(q, Entry{plan, layer, nullptr, true, src_head0, dst_head0, num_heads}, ready,
                     "kvx_queue_push_heads");
}

int kvx_queue_flush(kvx_queue* q) {
  if (!q) return fail(KVX_E_INVAL, "kvx_queue_flush: null queue");
  std::lock_guard<std::mutex> lk(q->mu);
  if (stream_capturing(q->stream)) return fail(KVX_E_INVAL, "kvx_queue_flush: the stream is capturing a graph");
  const int rc = flush(q);
  if (rc) drop_pending(q);
  return rc;
}

int kvx_queue_stats(const kvx_queue* q, int64_t* writes, int64_t* groups, int64_t* launches) {
  if (!q || !writes || !groups) return fail(KVX_E_INVAL, "kvx_queue_stats: null argument");
  kvx_queue* m = const_cast<kvx_queue*>(q);
  std::lock_guard<std::mutex> lk(m->mu);
  *writes = m->writes;
  *groups = m->groups;
  if (launches) *launches = m->launches;
  return KVX_OK;
}

int kvx_queue_destroy(kvx_queue* q) {
  if (!q) return KVX_OK;
  int rc;
  {
    std::lock_guard<std::mutex> lk(q->mu);
    rc = stream_capturing(q->stream) ? fail(KVX_E_INVAL, "kvx_queue_destroy: the stream is capturing a graph")
                                     : flush(q);
  }
  drop_pending(q);
  for (int i = 0; i < kInflight; ++i) (void)hipEventDestroy(q->done[i]);
  for (hipEvent_t e : q->all_events) (void)hipEventDestroy(e);
  (void)hipStreamDestroy(q->aux);
  delete q;
  return rc;
}

}  // extern "C"
