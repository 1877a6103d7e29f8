// libkvx transfer state machine (kvx_xfer_*): when each layer write of a
// request is issued and when the request is done, failed or expired.
//
// Sources: [PUSH] push-based NIXL connector post, "Implementierungsdetails"
// steps 1-3; [MORI] MoRIIO connector note §3.1, §3.2, §6 (full titles in
// kvx.h; the readings taken are listed in kvx_xfer.h).
//
// Device-side bookkeeping keeps queue packets and launches few: a layer save
// for many requests waits on the layer's event once (later writes on the
// same stream are ordered after it) and issues its writes as one batch
// (kvx_push_many); deferred writes of one save share one captured "gate"
// event, and a request's deferred layers go out as one batch; completion of
// issued writes is observed through one "mark" event recorded per poll
// behind every write issued since the previous poll (writes on one stream
// finish in order).

#include <hip/hip_runtime_api.h>

#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "kvx_internal.h"
#include "kvx_xfer.h"

namespace {

using namespace kvx;

enum LayerState : int8_t { kDeferred = 0, kIssued = 1, kDone = 2, kFailed = 3 };

struct Layer {
  LayerState st = kDeferred;
  double issued_at = 0;
  int32_t gate = -1;  // shared captured readiness of a deferred write (device mode)
};

struct Req {
  uint32_t attempt = 0;
  bool has_src = false, has_dst = false;
  int64_t ntok = 0;
  std::vector<int32_t> src, dst;
  const kvx_pool* consumer = nullptr;
  std::map<int32_t, Layer> layers;  // ordered by layer
  double deferred_since = -1;       // < 0: nothing deferred
  bool sealed = false;
  int64_t expected = 0;
  int32_t state = KVX_REQ_PENDING;
  bool reported = false;
  kvx_plan_t* plan = nullptr;
};

struct WriteRef {
  uint64_t id;
  uint32_t attempt;
  int32_t layer;
};

// A reference-counted event slot.
struct Sig {
  hipEvent_t ev = nullptr;
  int32_t refs = 0;
};

}  // namespace

struct kvx_xfer_s {
  const kvx_pool* producer = nullptr;
  kvx_xfer_config cfg{};
  hipStream_t stream = nullptr;
  bool host_only = false;
  bool keep_log = false;  // KVX_XFER_LOG
  std::map<uint64_t, Req> reqs;
  std::vector<WriteRef> log;  // issued writes, in order (KVX_XFER_LOG only)
  std::vector<Sig> sigs;
  std::vector<int32_t> free_sigs;
  std::vector<WriteRef> unmarked;                                  // issued since the last mark
  std::vector<std::pair<int32_t, std::vector<WriteRef>>> marks;    // mark -> writes it covers
  std::vector<std::pair<kvx_plan_t*, int32_t>> retired;            // plan freed when the mark fires
  mutable std::mutex mu;
};

namespace {

int sig_new(kvx_xfer* x, int32_t* idx) {
  int32_t i;
  if (!x->free_sigs.empty()) {
    i = x->free_sigs.back();
    x->free_sigs.pop_back();
  } else {
    x->sigs.push_back(Sig{});
    i = int32_t(x->sigs.size() - 1);
  }
  Sig& s = x->sigs[size_t(i)];
  if (!s.ev) {
    hipError_t e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      s.ev = nullptr;
      x->free_sigs.push_back(i);
      return fail_hip(e, "hipEventCreate(xfer)");
    }
  }
  s.refs = 1;
  *idx = i;
  return KVX_OK;
}

// Record a new signal behind everything enqueued on the stream so far.
int sig_mark(kvx_xfer* x, int32_t* idx) {
  int rc = sig_new(x, idx);
  if (rc != KVX_OK) return rc;
  hipError_t e = hipEventRecord(x->sigs[size_t(*idx)].ev, x->stream);
  if (e != hipSuccess) {
    x->sigs[size_t(*idx)].refs = 0;
    x->free_sigs.push_back(*idx);
    return fail_hip(e, "hipEventRecord(xfer)");
  }
  return KVX_OK;
}

void sig_unref(kvx_xfer* x, int32_t idx) {
  if (idx < 0) return;
  if (--x->sigs[size_t(idx)].refs == 0) x->free_sigs.push_back(idx);
}

// A request finished or was replaced: drop its gates and retire its plan.
// Its layer states stay for status queries.
void release_req(kvx_xfer* x, Req& r) {
  for (auto& kv : r.layers) {
    sig_unref(x, kv.second.gate);
    kv.second.gate = -1;
  }
  if (!r.plan) return;
  if (x->host_only) {
    plan_free_idle(r.plan);
  } else {
    // Work already enqueued on the stream (the plan upload, issued writes)
    // may still read the plan's descriptors: free it once a mark recorded
    // behind that work has fired.
    int32_t m = -1;
    if (sig_mark(x, &m) == KVX_OK) {
      x->retired.emplace_back(r.plan, m);
    } else {
      (void)hipStreamSynchronize(x->stream);
      plan_free_idle(r.plan);
    }
  }
  r.plan = nullptr;
}

// Find the request for (req, attempt): nullptr for a stale attempt; a newer
// attempt starts from a fresh record ([PUSH] step 2: re-sent and retried
// requests map to the right state).
Req* lookup(kvx_xfer* x, uint64_t id, uint32_t attempt, bool create) {
  auto it = x->reqs.find(id);
  if (it != x->reqs.end() && attempt < it->second.attempt) return nullptr;
  if (it == x->reqs.end() || attempt > it->second.attempt) {
    if (!create) return nullptr;
    if (it != x->reqs.end()) release_req(x, it->second);
    Req fresh;
    fresh.attempt = attempt;
    x->reqs[id] = std::move(fresh);
    return &x->reqs[id];
  }
  return &it->second;
}

// The outcome over every layer batch ([MORI] §6).
void settle(kvx_xfer* x, Req& r) {
  if (r.state != KVX_REQ_PENDING) return;
  int64_t done = 0;
  bool failed = false;
  for (auto& kv : r.layers) {
    failed |= kv.second.st == kFailed;
    done += kv.second.st == kDone;
  }
  if (failed)
    r.state = KVX_REQ_FAILED;
  else if (r.sealed && done == r.expected)
    r.state = KVX_REQ_DONE;
  if (r.state != KVX_REQ_PENDING) release_req(x, r);
}

// A layer write about to be issued.
struct Item {
  uint64_t id;
  Req* r;
  int32_t layer;
  Layer* ly;
};

// Issue layer writes, in order: one kvx_push_many on the stream, which is
// already ordered after their readiness (device mode); host-only mode only
// logs them.
int issue(kvx_xfer* x, const std::vector<Item>& items, double now) {
  if (items.empty()) return KVX_OK;
  if (!x->host_only) {
    std::vector<const kvx_plan_t*> plans;
    std::vector<int32_t> layers;
    plans.reserve(items.size());
    layers.reserve(items.size());
    for (const Item& it : items) {
      plans.push_back(it.r->plan);
      layers.push_back(it.layer);
    }
    int rc = kvx_push_many(plans.data(), layers.data(), int32_t(items.size()), nullptr, x->stream);
    if (rc != KVX_OK) return rc;
    for (const Item& it : items) x->unmarked.push_back(WriteRef{it.id, it.r->attempt, it.layer});
  }
  for (const Item& it : items) {
    it.ly->st = kIssued;
    it.ly->issued_at = now;
    if (x->keep_log) x->log.push_back(WriteRef{it.id, it.r->attempt, it.layer});
  }
  return KVX_OK;
}

// Both sides known: build the plan and issue every deferred layer in layer
// order ([PUSH] step 2: the second of registration and prefill triggers).
int start(kvx_xfer* x, uint64_t id, Req& r, double now) {
  if (r.state != KVX_REQ_PENDING || !r.has_src || !r.has_dst) return KVX_OK;
  if (!r.plan) {
    const int64_t so[2] = {0, int64_t(r.src.size())};
    const int64_t dof[2] = {0, int64_t(r.dst.size())};
    int rc = kvx_plan(x->producer, r.consumer, 1, &r.ntok, so, dof, r.src.data(), r.dst.data(),
                      x->host_only ? KVX_PLAN_HOST_ONLY : 0u, x->stream, &r.plan);
    if (rc != KVX_OK) {
      r.plan = nullptr;
      r.state = KVX_REQ_FAILED;
      release_req(x, r);
      return rc;
    }
  }
  // Every deferred layer, in layer order, in one batch behind the captured
  // readiness of each (layers saved together share one gate).
  std::vector<Item> items;
  int32_t waited = -1;
  for (auto& kv : r.layers) {
    if (kv.second.st != kDeferred) continue;
    const int32_t g = kv.second.gate;
    if (!x->host_only && g >= 0 && g != waited) {
      int rc = wait_event(x->sigs[size_t(g)].ev, x->stream);
      if (rc != KVX_OK) return rc;
      waited = g;
    }
    items.push_back(Item{id, &r, kv.first, &kv.second});
  }
  int rc = issue(x, items, now);
  if (rc != KVX_OK) return rc;
  r.deferred_since = -1;
  return KVX_OK;
}

void set(int32_t* p, int32_t v) {
  if (p) *p = v;
}

int save_many(kvx_xfer* x, int32_t layer, hipEvent_t ready, int64_t n, const uint64_t* ids,
              const uint32_t* attempts, double now, int32_t* accepted) {
  // Classify first, so that the stream waits on `ready` once and the
  // deferred writes share one captured gate.
  std::vector<Req*> take(size_t(n), nullptr);
  int64_t n_issue = 0, n_defer = 0;
  for (int64_t i = 0; i < n; ++i) {
    set(accepted ? accepted + i : nullptr, 0);
    Req* r = lookup(x, ids[i], attempts[i], false);
    if (!r || r->state != KVX_REQ_PENDING || r->sealed) continue;
    set(accepted ? accepted + i : nullptr, 1);
    if (r->layers.count(layer)) continue;
    for (int64_t j = 0; j < i; ++j)  // the same request twice in one call counts once
      if (take[size_t(j)] == r) r = nullptr;
    if (!r) continue;
    take[size_t(i)] = r;
    if (r->plan)
      ++n_issue;
    else
      ++n_defer;
  }
  int32_t gate = -1;
  if (!x->host_only && ready && (n_issue || n_defer)) {
    hipError_t q = hipEventQuery(ready);
    if (q == hipErrorNotReady) {
      hipError_t e = hipStreamWaitEvent(x->stream, ready, 0);
      if (e != hipSuccess) return fail_hip(e, "hipStreamWaitEvent(ready)");
      if (n_defer) {
        // Capture the readiness now, so the caller may reuse `ready`.
        int rc = sig_mark(x, &gate);
        if (rc != KVX_OK) return rc;
        x->sigs[size_t(gate)].refs = int32_t(n_defer);
      }
    } else if (q != hipSuccess) {
      return fail_hip(q, "hipEventQuery(ready)");
    }
  }
  std::vector<Item> items;
  items.reserve(size_t(n_issue));
  for (int64_t i = 0; i < n; ++i) {
    Req* r = take[size_t(i)];
    if (!r) continue;
    Layer& ly = r->layers[layer];
    if (r->plan) {
      items.push_back(Item{ids[i], r, layer, &ly});  // stream order already follows `ready`
    } else {
      ly.st = kDeferred;
      ly.gate = gate;
      if (r->deferred_since < 0) r->deferred_since = now;
    }
  }
  return issue(x, items, now);
}

}  // namespace

extern "C" {

int kvx_xfer_create(const kvx_pool* producer, const kvx_xfer_config* cfg, hipStream_t stream, kvx_xfer** out) {
  if (!producer || !out) return fail(KVX_E_INVAL, "kvx_xfer_create: null argument");
  kvx_xfer* x = new (std::nothrow) kvx_xfer;
  if (!x) return fail(KVX_E_NOMEM, "kvx_xfer_create: out of host memory");
  x->producer = producer;
  x->cfg = cfg ? *cfg : kvx_xfer_config{60.0, 30.0, 0u};
  if (x->cfg.flags & ~(KVX_XFER_HOST_ONLY | KVX_XFER_LOG)) {
    const uint32_t f = x->cfg.flags;
    delete x;
    return fail(KVX_E_INVAL, "kvx_xfer_create: unknown flags 0x%x", f);
  }
  x->host_only = (x->cfg.flags & KVX_XFER_HOST_ONLY) != 0;
  x->keep_log = (x->cfg.flags & KVX_XFER_LOG) != 0;
  x->stream = stream;
  *out = x;
  return KVX_OK;
}

void kvx_xfer_destroy(kvx_xfer* x) {
  if (!x) return;
  if (!x->host_only) (void)hipStreamSynchronize(x->stream);
  for (auto& kv : x->reqs)
    if (kv.second.plan) plan_free_idle(kv.second.plan);
  for (auto& rp : x->retired) plan_free_idle(rp.first);
  for (Sig& s : x->sigs)
    if (s.ev) (void)hipEventDestroy(s.ev);
  delete x;
}

int kvx_xfer_register(kvx_xfer* x, uint64_t id, uint32_t attempt, const kvx_pool* consumer,
                      const int32_t* dst_ids, int64_t n, double now, int32_t* accepted) {
  if (!x || !consumer || n < 0 || (n > 0 && !dst_ids)) return fail(KVX_E_INVAL, "kvx_xfer_register: bad argument");
  std::lock_guard<std::mutex> lk(x->mu);
  set(accepted, 0);
  try {
    Req* r = lookup(x, id, attempt, true);
    if (!r || r->state != KVX_REQ_PENDING || r->has_dst) return KVX_OK;
    r->dst.assign(dst_ids, dst_ids + n);
    r->consumer = consumer;
    r->has_dst = true;
    set(accepted, 1);
    return start(x, id, *r, now);
  } catch (const std::bad_alloc&) {
    return fail(KVX_E_NOMEM, "kvx_xfer_register: out of host memory");
  }
}

int kvx_xfer_prefill(kvx_xfer* x, uint64_t id, uint32_t attempt, int64_t num_tokens, const int32_t* src_ids,
                     int64_t n, double now, int32_t* accepted) {
  if (!x || num_tokens < 0 || n < 0 || (n > 0 && !src_ids))
    return fail(KVX_E_INVAL, "kvx_xfer_prefill: bad argument");
  std::lock_guard<std::mutex> lk(x->mu);
  set(accepted, 0);
  try {
    Req* r = lookup(x, id, attempt, true);
    if (!r || r->state != KVX_REQ_PENDING || r->has_src) return KVX_OK;
    r->src.assign(src_ids, src_ids + n);
    r->ntok = num_tokens;
    r->has_src = true;
    set(accepted, 1);
    return start(x, id, *r, now);
  } catch (const std::bad_alloc&) {
    return fail(KVX_E_NOMEM, "kvx_xfer_prefill: out of host memory");
  }
}

int kvx_xfer_save_layer(kvx_xfer* x, uint64_t id, uint32_t attempt, int32_t layer, hipEvent_t ready, double now,
                        int32_t* accepted) {
  return kvx_xfer_save_layer_many(x, layer, ready, 1, &id, &attempt, now, accepted);
}

int kvx_xfer_save_layer_many(kvx_xfer* x, int32_t layer, hipEvent_t ready, int64_t n, const uint64_t* reqs,
                             const uint32_t* attempts, double now, int32_t* accepted) {
  if (!x || n < 0 || (n > 0 && (!reqs || !attempts))) return fail(KVX_E_INVAL, "kvx_xfer_save_layer: bad argument");
  if (layer < 0 || layer >= x->producer->g.L)
    return fail(KVX_E_RANGE, "kvx_xfer_save_layer: layer %d outside [0,%d)", layer, x->producer->g.L);
  std::lock_guard<std::mutex> lk(x->mu);
  try {
    return save_many(x, layer, ready, n, reqs, attempts, now, accepted);
  } catch (const std::bad_alloc&) {
    return fail(KVX_E_NOMEM, "kvx_xfer_save_layer: out of host memory");
  }
}

int kvx_xfer_seal(kvx_xfer* x, uint64_t id, uint32_t attempt, int32_t* accepted) {
  if (!x) return fail(KVX_E_INVAL, "kvx_xfer_seal: null argument");
  std::lock_guard<std::mutex> lk(x->mu);
  set(accepted, 0);
  Req* r = lookup(x, id, attempt, false);
  if (!r || r->state != KVX_REQ_PENDING || r->sealed) return KVX_OK;
  r->sealed = true;
  r->expected = int64_t(r->layers.size());
  set(accepted, 1);
  settle(x, *r);
  return KVX_OK;
}

int kvx_xfer_poll(kvx_xfer* x, double now) {
  if (!x) return fail(KVX_E_INVAL, "kvx_xfer_poll: null argument");
  std::lock_guard<std::mutex> lk(x->mu);
  try {
    if (!x->host_only) {
      // marks that fired: every write behind them is done
      for (size_t i = 0; i < x->marks.size();) {
        hipError_t q = hipEventQuery(x->sigs[size_t(x->marks[i].first)].ev);
        if (q == hipErrorNotReady) {
          ++i;
          continue;
        }
        if (q != hipSuccess) return fail_hip(q, "hipEventQuery(xfer mark)");
        for (const WriteRef& w : x->marks[i].second) {
          auto it = x->reqs.find(w.id);
          if (it == x->reqs.end() || it->second.attempt != w.attempt) continue;
          auto ly = it->second.layers.find(w.layer);
          if (ly != it->second.layers.end() && ly->second.st == kIssued) ly->second.st = kDone;
        }
        sig_unref(x, x->marks[i].first);
        x->marks[i] = std::move(x->marks.back());
        x->marks.pop_back();
      }
      // one mark behind the writes issued since the previous poll
      if (!x->unmarked.empty()) {
        int32_t m = -1;
        int rc = sig_mark(x, &m);
        if (rc != KVX_OK) return rc;
        x->marks.emplace_back(m, std::move(x->unmarked));
        x->unmarked.clear();
      }
      // retired plans whose enqueued work has finished
      for (size_t i = 0; i < x->retired.size();) {
        hipError_t q = hipEventQuery(x->sigs[size_t(x->retired[i].second)].ev);
        if (q == hipSuccess) {
          plan_free_idle(x->retired[i].first);
          sig_unref(x, x->retired[i].second);
          x->retired[i] = x->retired.back();
          x->retired.pop_back();
        } else if (q == hipErrorNotReady) {
          ++i;
        } else {
          return fail_hip(q, "hipEventQuery(xfer retired plan)");
        }
      }
    }
    for (auto& kv : x->reqs) {
      Req& r = kv.second;
      if (r.state != KVX_REQ_PENDING) continue;
      if (r.deferred_since >= 0 && now - r.deferred_since >= x->cfg.defer_timeout_s) {
        r.state = KVX_REQ_EXPIRED;
        release_req(x, r);
        continue;
      }
      for (auto& l : r.layers)
        if (l.second.st == kIssued && now - l.second.issued_at >= x->cfg.transfer_timeout_s) l.second.st = kFailed;
      settle(x, r);
    }
    return KVX_OK;
  } catch (const std::bad_alloc&) {
    return fail(KVX_E_NOMEM, "kvx_xfer_poll: out of host memory");
  }
}

int kvx_xfer_complete(kvx_xfer* x, uint64_t id, uint32_t attempt, int32_t layer, int32_t ok) {
  if (!x) return fail(KVX_E_INVAL, "kvx_xfer_complete: null argument");
  if (ok && !x->host_only)
    return fail(KVX_E_INVAL, "kvx_xfer_complete: completion is observed by kvx_xfer_poll on the device");
  std::lock_guard<std::mutex> lk(x->mu);
  Req* r = lookup(x, id, attempt, false);
  if (!r) return KVX_OK;
  auto it = r->layers.find(layer);
  if (it == r->layers.end() || it->second.st != kIssued) return KVX_OK;
  it->second.st = ok ? kDone : kFailed;
  settle(x, *r);
  return KVX_OK;
}

int kvx_xfer_status(const kvx_xfer* x, uint64_t id, uint32_t* attempt, int32_t* state) {
  if (!x || !attempt || !state) return fail(KVX_E_INVAL, "kvx_xfer_status: null argument");
  std::lock_guard<std::mutex> lk(x->mu);
  auto it = x->reqs.find(id);
  if (it == x->reqs.end()) return fail(KVX_E_RANGE, "kvx_xfer_status: unknown request");
  *attempt = it->second.attempt;
  *state = it->second.state;
  return KVX_OK;
}

int kvx_xfer_pop_finished(kvx_xfer* x, uint64_t* reqs, uint32_t* attempts, int32_t* states, int64_t cap,
                          int64_t* n) {
  if (!x || !n || (cap > 0 && (!reqs || !attempts || !states)))
    return fail(KVX_E_INVAL, "kvx_xfer_pop_finished: bad argument");
  std::lock_guard<std::mutex> lk(x->mu);
  int64_t k = 0;
  for (auto& kv : x->reqs) {
    if (k >= cap) break;
    Req& r = kv.second;
    if (r.state == KVX_REQ_PENDING || r.reported) continue;
    r.reported = true;
    reqs[k] = kv.first;
    attempts[k] = r.attempt;
    states[k] = r.state;
    ++k;
  }
  *n = k;
  return KVX_OK;
}

int kvx_xfer_recompute_blocks(const kvx_xfer* x, uint64_t id, int32_t* out, int64_t cap, int64_t* n) {
  if (!x || !n) return fail(KVX_E_INVAL, "kvx_xfer_recompute_blocks: null argument");
  std::lock_guard<std::mutex> lk(x->mu);
  auto it = x->reqs.find(id);
  if (it == x->reqs.end()) return fail(KVX_E_RANGE, "kvx_xfer_recompute_blocks: unknown request");
  const Req& r = it->second;
  const bool lost = r.state == KVX_REQ_FAILED || r.state == KVX_REQ_EXPIRED;
  const int64_t cnt = lost && r.has_dst ? int64_t(r.dst.size()) : 0;
  if (out && cap >= cnt)
    for (int64_t i = 0; i < cnt; ++i) out[i] = r.dst[size_t(i)];
  *n = cnt;
  return KVX_OK;
}

int kvx_xfer_issued(const kvx_xfer* x, int64_t first, uint64_t* reqs, uint32_t* attempts, int32_t* layers,
                    int64_t cap, int64_t* n) {
  if (!x || !n || first < 0 || (cap > 0 && (!reqs || !attempts || !layers)))
    return fail(KVX_E_INVAL, "kvx_xfer_issued: bad argument");
  if (!x->keep_log) return fail(KVX_E_INVAL, "kvx_xfer_issued: created without KVX_XFER_LOG");
  std::lock_guard<std::mutex> lk(x->mu);
  int64_t k = 0;
  for (int64_t i = first; i < int64_t(x->log.size()) && k < cap; ++i, ++k) {
    reqs[k] = x->log[size_t(i)].id;
    attempts[k] = x->log[size_t(i)].attempt;
    layers[k] = x->log[size_t(i)].layer;
  }
  *n = k;
  return KVX_OK;
}

int kvx_xfer_forget(kvx_xfer* x, uint64_t id) {
  if (!x) return fail(KVX_E_INVAL, "kvx_xfer_forget: null argument");
  std::lock_guard<std::mutex> lk(x->mu);
  auto it = x->reqs.find(id);
  if (it == x->reqs.end()) return fail(KVX_E_RANGE, "kvx_xfer_forget: unknown request");
  if (it->second.state == KVX_REQ_PENDING) return fail(KVX_E_INVAL, "kvx_xfer_forget: request still pending");
  release_req(x, it->second);
  x->reqs.erase(it);
  return KVX_OK;
}

}  // extern "C"
