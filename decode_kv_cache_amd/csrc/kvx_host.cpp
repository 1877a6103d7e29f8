// libkvx host side: status strings, pool registry, transfer planning (run
// merge, per-region triples, device work list) and plan lifetime.
//
// Sources: [PUSH] push-based NIXL connector post, [MORI] MoRIIO connector
// note, [BIDIR] bidirectional KV transfer post (full titles in kvx.h).

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "kvx_arena.h"
#include "kvx_internal.h"

namespace kvx {

static thread_local std::string t_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_err = buf;
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  return fail(KVX_E_HIP, "%s: %s (%d)", what, hipGetErrorString(e), int(e));
}

// True while `s` is capturing a graph.  An event query or a host wait on
// another thread's behalf would then invalidate the capture, so the waits
// below take the graph path instead.
static bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st == hipStreamCaptureStatusActive;
}

static int wait_event_on(hipEvent_t ev, hipStream_t s, bool cap) {
  if (!ev) return KVX_OK;
  if (!cap) {
    // An event whose work has already completed needs no wait: skipping it
    // saves the queue a barrier packet (several microseconds per layer).
    hipError_t q = hipEventQuery(ev);
    if (q == hipSuccess) return KVX_OK;
    if (q != hipErrorNotReady) return fail_hip(q, "hipEventQuery(ready)");
  }
  // Under capture the wait becomes a graph dependency (the event must have
  // been recorded in the same capture).
  hipError_t e = hipStreamWaitEvent(s, ev, 0);
  if (e != hipSuccess) return fail_hip(e, "hipStreamWaitEvent(ready)");
  return KVX_OK;
}

int wait_event(hipEvent_t ev, hipStream_t s) { return wait_event_on(ev, s, ev && capturing(s)); }

bool stream_capturing(hipStream_t s) { return capturing(s); }

int enqueue_waits(kvx_plan_t* p, hipEvent_t ready, hipStream_t s) {
  const bool seen = p->upload_seen.load(std::memory_order_acquire);
  const bool cap = (ready || !seen) && capturing(s);
  int rc = wait_event_on(ready, s, cap);
  if (rc) return rc;
  if (seen) return KVX_OK;
  if (cap)  // no query of the upload event is allowed inside the capture
    return fail(KVX_E_INVAL,
                "plan's upload not yet observed complete inside a graph capture: call kvx_plan_wait before "
                "capturing");
  hipError_t q = hipEventQuery(p->upload_ev);
  if (q == hipSuccess) {
    p->upload_seen.store(true, std::memory_order_release);
  } else if (q == hipErrorNotReady) {
    hipError_t e = hipStreamWaitEvent(s, p->upload_ev, 0);
    if (e != hipSuccess) return fail_hip(e, "hipStreamWaitEvent(upload)");
  } else {
    return fail_hip(q, "hipEventQuery(upload)");
  }
  return KVX_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, what);
  return KVX_OK;
}

static int64_t pad16(int64_t x) { return (x + 15) / 16 * 16; }

// Work-list arena, one per device (RangeArena): chunks of at least 64 MiB
// from hipMalloc, kept mapped until the process ends.  Freeing a work list
// never calls hipFree, which synchronizes the whole device: a finished
// request's plan is released while other work runs (kvx_xfer_poll).
constexpr int kMaxDevices = 64;
constexpr size_t kArenaChunk = size_t(64) << 20;
constexpr size_t kArenaChunkAlign = size_t(2) << 20;

static RangeArena* make_arenas() {
  // Never destroyed: a plan may be freed while the process shuts down.
  RangeArena* a = static_cast<RangeArena*>(::operator new(sizeof(RangeArena) * kMaxDevices));
  for (int d = 0; d < kMaxDevices; ++d) new (a + d) RangeArena(kArenaChunk, kArenaChunkAlign);
  return a;
}
static RangeArena* const g_arena = make_arenas();

static int hip_chunk(size_t bytes, void** out) { return int(hipMalloc(out, bytes)); }

int desc_alloc(size_t bytes, void** out, int* device) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(KVX_E_UNSUPPORTED, "kvx_plan: device %d beyond %d", dev, kMaxDevices);
  *device = dev;
  const size_t n = (bytes + 255) / 256 * 256;
  const int rc = g_arena[dev].alloc(n, hip_chunk, out);
  if (rc == 0) return KVX_OK;
  e = hipError_t(rc);
  return e == hipErrorOutOfMemory ? fail(KVX_E_NOMEM, "kvx_plan: device work list (%zu B)", n)
                                  : fail_hip(e, "hipMalloc(work-list chunk)");
}

void desc_free(void* p, size_t bytes, int device) {
  if (p && device >= 0 && device < kMaxDevices) (void)g_arena[device].release(p, (bytes + 255) / 256 * 256);
}

void plan_free_idle(kvx_plan_t* p) {
  if (!p) return;
  if (p->upload_ev) {
    (void)hipEventSynchronize(p->upload_ev);
    (void)hipEventDestroy(p->upload_ev);
  }
  if (!p->in_scratch) desc_free(p->dev_buf, p->dev_bytes, p->device);
  delete p;
}

}  // namespace kvx

using namespace kvx;

extern "C" {

int32_t kvx_abi_version(void) { return KVX_ABI_VERSION; }

const char* kvx_status_str(int s) {
  switch (s) {
    case KVX_OK: return "KVX_OK";
    case KVX_E_INVAL: return "KVX_E_INVAL";
    case KVX_E_RANGE: return "KVX_E_RANGE";
    case KVX_E_DUPDST: return "KVX_E_DUPDST";
    case KVX_E_MISMATCH: return "KVX_E_MISMATCH";
    case KVX_E_UNSUPPORTED: return "KVX_E_UNSUPPORTED";
    case KVX_E_NOMEM: return "KVX_E_NOMEM";
    case KVX_E_HIP: return "KVX_E_HIP";
    default: return "KVX_E_UNKNOWN";
  }
}

const char* kvx_last_error(void) { return t_err.c_str(); }

// [MORI] §3.1: the consumer takes prompt - computed - 1 tokens and recomputes
// the final prompt token itself.
int64_t kvx_tokens_to_move(int64_t prompt_len, int64_t num_computed) {
  int64_t n = prompt_len - num_computed - 1;
  return n > 0 ? n : 0;
}

// [BIDIR] "KV-Recompute-Schwellenwert": pull at or above the threshold.
int32_t kvx_should_reuse(int64_t reusable_tokens, int64_t threshold) {
  return reusable_tokens >= threshold ? 1 : 0;
}

int kvx_pool_create(const kvx_pool_desc* d, kvx_pool** out) {
  if (!d || !out) return fail(KVX_E_INVAL, "kvx_pool_create: null argument");
  if (d->num_layers < 1 || d->num_blocks < 1 || d->block_size < 1 || d->num_heads < 1 ||
      d->head_dim < 1)
    return fail(KVX_E_INVAL, "kvx_pool_create: counts must be >= 1");
  if (d->elem_bytes != 1 && d->elem_bytes != 2 && d->elem_bytes != 4)
    return fail(KVX_E_INVAL, "kvx_pool_create: elem_bytes %d not in {1,2,4}", d->elem_bytes);
  if (d->layout != KVX_NHD && d->layout != KVX_HND)
    return fail(KVX_E_INVAL, "kvx_pool_create: unknown layout %d", d->layout);
  if (!d->k_base) return fail(KVX_E_INVAL, "kvx_pool_create: null k_base array");
  const bool latent = d->v_base == nullptr;  // one region per layer (MLA)
  if (latent && d->v_scale)
    return fail(KVX_E_INVAL, "kvx_pool_create: v_scale set for a pool without a V region");
  if (!latent && (d->k_scale == nullptr) != (d->v_scale == nullptr))
    return fail(KVX_E_INVAL, "kvx_pool_create: k_scale and v_scale must both be set or both NULL");
  if (d->sliding_window < 0) return fail(KVX_E_INVAL, "kvx_pool_create: negative sliding_window");
  if (d->block_size > 32768)
    return fail(KVX_E_UNSUPPORTED, "kvx_pool_create: block_size %d above 32768", d->block_size);
  if ((int64_t(d->head_dim) * d->elem_bytes) % 16)
    return fail(KVX_E_UNSUPPORTED, "kvx_pool_create: head_dim*elem_bytes=%lld not a multiple of 16",
                (long long)(int64_t(d->head_dim) * d->elem_bytes));
  // The head-slice kernel addresses inside one block with 32-bit offsets.
  const int64_t blk = int64_t(d->block_size) * d->num_heads * d->head_dim * d->elem_bytes;
  if (blk > INT32_MAX)
    return fail(KVX_E_UNSUPPORTED, "kvx_pool_create: block of %lld bytes (2^31 or more)", (long long)blk);
  kvx_pool* p = new (std::nothrow) kvx_pool;
  if (!p) return fail(KVX_E_NOMEM, "kvx_pool_create: out of host memory");
  Geom& g = p->g;
  g.L = d->num_layers;
  g.NB = d->num_blocks;
  g.BS = d->block_size;
  g.H = d->num_heads;
  g.D = d->head_dim;
  g.E = d->elem_bytes;
  g.layout = d->layout;
  g.nreg = latent ? 1 : 2;
  g.window = d->sliding_window;
  g.scales = d->k_scale != nullptr;
  try {
    for (int l = 0; l < g.L; ++l) {
      void* k = d->k_base[l];
      void* v = latent ? k : d->v_base[l];
      if (!k || !v) {
        delete p;
        return fail(KVX_E_INVAL, "kvx_pool_create: null base for layer %d", l);
      }
      if ((uintptr_t(k) | uintptr_t(v)) & 15) {
        delete p;
        return fail(KVX_E_UNSUPPORTED, "kvx_pool_create: layer %d base not 16-byte aligned", l);
      }
      g.k.push_back(k);
      if (!latent) g.v.push_back(v);
      if (g.scales) {
        float* ks = d->k_scale[l];
        float* vs = latent ? ks : d->v_scale[l];
        if (!ks || !vs) {
          delete p;
          return fail(KVX_E_INVAL, "kvx_pool_create: null scale pointer for layer %d", l);
        }
        if ((uintptr_t(ks) | uintptr_t(vs)) & 3) {
          delete p;
          return fail(KVX_E_UNSUPPORTED, "kvx_pool_create: layer %d scales not 4-byte aligned", l);
        }
        g.ks.push_back(ks);
        if (!latent) g.vs.push_back(vs);
      }
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(KVX_E_NOMEM, "kvx_pool_create: out of host memory");
  }
  *out = p;
  return KVX_OK;
}

int kvx_state_pool_create(const kvx_state_pool_desc* d, kvx_pool** out) {
  if (!d || !out) return fail(KVX_E_INVAL, "kvx_state_pool_create: null argument");
  if (d->num_layers < 1 || d->num_slots < 1)
    return fail(KVX_E_INVAL, "kvx_state_pool_create: counts must be >= 1");
  if (!d->base[0] || !d->base[1]) return fail(KVX_E_INVAL, "kvx_state_pool_create: null base array");
  for (int r = 0; r < 2; ++r)
    if (d->slot_bytes[r] < 16 || d->slot_bytes[r] % 16)
      return fail(KVX_E_UNSUPPORTED, "kvx_state_pool_create: slot_bytes[%d]=%lld not a positive multiple of 16",
                  r, (long long)d->slot_bytes[r]);
  kvx_pool* p = new (std::nothrow) kvx_pool;
  if (!p) return fail(KVX_E_NOMEM, "kvx_state_pool_create: out of host memory");
  Geom& g = p->g;
  g.state = true;
  g.L = d->num_layers;
  g.NB = d->num_slots;
  g.nreg = 2;
  g.slot_bytes[0] = d->slot_bytes[0];
  g.slot_bytes[1] = d->slot_bytes[1];
  try {
    for (int l = 0; l < g.L; ++l) {
      void* b0 = d->base[0][l];
      void* b1 = d->base[1][l];
      if (!b0 || !b1) {
        delete p;
        return fail(KVX_E_INVAL, "kvx_state_pool_create: null base for layer %d", l);
      }
      if ((uintptr_t(b0) | uintptr_t(b1)) & 15) {
        delete p;
        return fail(KVX_E_UNSUPPORTED, "kvx_state_pool_create: layer %d base not 16-byte aligned", l);
      }
      g.k.push_back(b0);
      g.v.push_back(b1);
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(KVX_E_NOMEM, "kvx_state_pool_create: out of host memory");
  }
  *out = p;
  return KVX_OK;
}

void kvx_pool_destroy(kvx_pool* p) { delete p; }

}  // extern "C"

namespace {

// Append a byte range to the triple list, merging it into the previous triple
// when both the source and the destination continue without a gap.
void emit(std::vector<kvx_triple>& t, int64_t so, int64_t dso, int64_t len) {
  if (!t.empty()) {
    kvx_triple& b = t.back();
    if (b.src_off + b.len == so && b.dst_off + b.len == dso) {
      b.len += len;
      return;
    }
  }
  t.push_back(kvx_triple{so, dso, len});
}

// Triples of one (layer, K/V) region, in plan order ([MORI] §6: the
// (local offset, remote offset, size) list of one batch call, adjacent
// blocks merged).  Each planned block (or, with different block sizes, each
// piece of a token range inside one source and one destination block)
// contributes its token rows: one range in NHD, one range per head in HND;
// `emit` merges ranges that continue on both sides, so consecutive blocks of
// a run become one range.
void build_triples(kvx_plan_t* p) {
  const Geom& gs = p->src;
  const Geom& gd = p->dst;
  const int64_t tb = gs.token_bytes(), rb = gs.row_bytes();
  p->triples[0].reserve(p->blocks.size() * (gs.layout == KVX_NHD ? 1 : size_t(gs.H)));
  for (const BlockPair& b : p->blocks) {
    const int64_t ss = slot_src(b.slots), ds = slot_dst(b.slots);
    const int64_t sbase = int64_t(b.src) * gs.block_bytes(), dbase = int64_t(b.dst) * gd.block_bytes();
    if (gs.layout == KVX_NHD) {
      emit(p->triples[0], sbase + ss * tb, dbase + ds * tb, int64_t(b.nslots) * tb);
    } else {
      for (int h = 0; h < gs.H; ++h)
        emit(p->triples[0], sbase + (int64_t(h) * gs.BS + ss) * rb, dbase + (int64_t(h) * gd.BS + ds) * rb,
             int64_t(b.nslots) * rb);
    }
  }
}

// Launch shape for a plan, from its triples, as measured on MI355X (every
// shape side by side on the same pools, and plain copies of 12 MiB to 4 GiB
// per launch in each shape).  "Fill" is the plan's bytes over the capacity
// of the 32 KiB pieces covering its triples; n32 is the number of those
// pieces in one layer's launch.
//  - Runs that fill 32 KiB pieces to at least 90% (whole blocks of 32 KiB,
//    long state slots) in a launch of about one round of one-wave
//    workgroups per SIMD copy fastest as one-wave workgroups: every load of
//    a piece issued before its first store, the launch's reads and writes
//    largely in two phases.  32 KiB pieces from 608 to 1312 of them (19 to
//    41 MiB read per launch), 16 KiB pieces below that.
//  - Larger launches (past about 42 MiB read) and runs that fill pieces
//    less (blocks of 16 KiB or smaller, ragged run ends) stream fastest as
//    4 KiB pieces of four-wave workgroups: a plain copy in that shape
//    reaches 6.5 TB/s read+write from 256 MiB per launch, where one-wave
//    32 KiB pieces stay near 5.3-5.6.
//  - So do plans whose launches overlap one another (KVX_PLAN_OVERLAP): the
//    next launch's small workgroups fill in behind this one's last ones
//    (the 64-layer Qwen3-32B-shaped push over two side streams: 11.7 us
//    per layer against 13.0 on one stream with one-wave pieces, and 13.7
//    with one-wave pieces on two streams).
int32_t pick_shape(kvx_plan_t* p) {
  int64_t n32 = 0, bytes = 0;
  for (int32_t r = 0; r < p->nlists; ++r)
    for (const kvx_triple& t : p->triples[r]) {
      n32 += (t.len + 32767) / 32768;
      bytes += t.len;
    }
  if (p->nlists == 1) {  // every region copies the shared list
    n32 *= p->nreg;
    bytes *= p->nreg;
  }
  p->n32 = n32;
  if (p->overlap || n32 == 0 || n32 > kLongMaxPieces || bytes * 10 < n32 * 32768 * 9) return kShapeFine;
  return n32 >= kLongMinPieces ? kShapeLong : kShapeLongSmall;
}

// Indices of a triple list in destination-offset order: an LSD radix sort of
// (offset, index) pairs on 11-bit digits, skipping the digits every offset
// shares (offsets below 4 GiB take three passes).  The comparison sort it
// replaces took 1.5 ms for the batched push's 27k triples.
std::vector<int32_t> dst_order(const std::vector<kvx_triple>& tr) {
  constexpr int kBits = 11;
  constexpr uint64_t kMask = (uint64_t(1) << kBits) - 1;
  const size_t n = tr.size();
  std::vector<std::pair<uint64_t, int32_t>> a(n), b(n);
  uint64_t any = 0, all = ~uint64_t(0);
  for (size_t i = 0; i < n; ++i) {
    a[i] = {uint64_t(tr[i].dst_off), int32_t(i)};
    any |= a[i].first;
    all &= a[i].first;
  }
  std::vector<uint32_t> count(size_t(1) << kBits);
  for (int shift = 0; shift < 64; shift += kBits) {
    if ((((any ^ all) >> shift) & kMask) == 0) continue;  // this digit is the same in every offset
    std::fill(count.begin(), count.end(), 0u);
    for (const auto& e : a) ++count[(e.first >> shift) & kMask];
    uint32_t sum = 0;
    for (uint32_t& c : count) {
      const uint32_t k = c;
      c = sum;
      sum += k;
    }
    for (const auto& e : a) b[count[(e.first >> shift) & kMask]++] = e;
    a.swap(b);
  }
  std::vector<int32_t> order(n);
  for (size_t i = 0; i < n; ++i) order[i] = a[i].second;
  return order;
}

// First run of each group of kRunGroupChunks chunks of a run table's flat
// space: the run that holds the group's first 16-byte unit.
std::vector<uint32_t> run_index(const std::vector<RunRec>& runs, uint32_t total16) {
  const uint64_t chunks = (uint64_t(total16) + kRunChunk16 - 1) / kRunChunk16;
  const uint64_t groups = (chunks + kRunGroupChunks - 1) / kRunGroupChunks;
  std::vector<uint32_t> g(size_t(groups), 0);
  size_t r = 0;
  for (uint64_t k = 0; k < groups; ++k) {
    const uint64_t target = k * uint64_t(kRunGroupChunks) * kRunChunk16;
    while (r + 1 < runs.size() && uint64_t(runs[r].start16) + runs[r].len16 <= target) ++r;
    g[size_t(k)] = uint32_t(r);
  }
  return g;
}

// Whether a plan can keep run tables: streaming launches, one triple list
// shared by the regions, and regions (hence staging) below 4 GiB, so that
// every byte offset fits 32 bits.
bool runs_eligible(const kvx_plan_t* p) {
  const int64_t lim = int64_t(1) << 32;
  return p->want_runs && p->shape == kShapeFine && p->nlists == 1 &&
         int64_t(p->src.NB) * p->src.block_bytes() < lim && int64_t(p->dst.NB) * p->dst.block_bytes() < lim;
}

// Run tables of the shared triple list (KVX_PLAN_RUNS): in plan order with
// each run's staging offset as its flat position (pack, unpack), and in
// destination order (push; the order streaming pieces take, for the same
// reason).
void build_runs(kvx_plan_t* p) {
  const std::vector<kvx_triple>& tr = p->triples[0];
  const size_t n = tr.size();
  p->runs_plan.resize(n);
  uint32_t pos = 0;
  for (size_t i = 0; i < n; ++i) {
    const kvx_triple& t = tr[i];
    p->runs_plan[i] = RunRec{uint32_t(t.src_off / 16), uint32_t(t.dst_off / 16), uint32_t(t.len / 16), pos};
    pos += uint32_t(t.len / 16);
  }
  p->run_total16 = pos;
  p->payload[0] = p->payload[1] = int64_t(pos) * 16;
  const std::vector<int32_t> order = dst_order(tr);
  p->runs_dst.resize(n);
  pos = 0;
  for (size_t k = 0; k < n; ++k) {
    RunRec r = p->runs_plan[size_t(order[k])];
    r.start16 = pos;
    pos += r.len16;
    p->runs_dst[k] = r;
  }
  p->gidx_plan = run_index(p->runs_plan, p->run_total16);
  p->gidx_dst = run_index(p->runs_dst, p->run_total16);
  p->runs_mode = true;
}

// Split each triple list into workgroup-sized pieces and give each its
// offset in its region's staging (the exclusive prefix of the triple
// lengths).  Pieces of list r carry r as their region tag.  A plan that
// asked for run tables and can keep them gets those instead.
void build_pieces(kvx_plan_t* p) {
  p->shape = pick_shape(p);
  if (runs_eligible(p)) {
    build_runs(p);
    return;
  }
  const int64_t piece = shape_piece_bytes(p->shape);
  // Streaming launches take their pieces in destination order: the
  // workgroups resident at any moment then write a narrow address range
  // (measured side by side against plan order: the multi-turn fp8 layer 15%
  // faster, the MLA layer 10%, the batched push 7%, large attention layers
  // 6%, unpack 5.5%; pack unchanged).  One-wave launches keep plan order: a
  // launch of about one round issues every piece at once, and in plan order
  // it is as fast or faster (state slots 4%).  A one-wave plan also keeps its
  // pieces in destination order (stream_pieces) for the launches that
  // stream them as 4 KiB chunks, several layers at once: all 64 layers of
  // the Qwen3-32B-shaped push in one kvx_push_many call run 4% faster so.
  // The triples of one list write disjoint destination ranges, so ordering
  // the triples orders their pieces; each piece keeps its staging offset
  // (the exclusive prefix of the triple lengths in plan order), so the
  // staging layout does not depend on it.
  const bool by_dst = p->shape == kShapeFine;
  std::vector<int64_t> stg;
  std::vector<int32_t> order;
  size_t count = 0;
  for (int32_t r = 0; r < p->nlists; ++r)
    for (const kvx_triple& t : p->triples[r]) count += size_t((t.len + piece - 1) / piece);
  p->pieces.reserve(count);
  for (int32_t r = 0; r < p->nlists; ++r) {
    const std::vector<kvx_triple>& tr = p->triples[r];
    stg.assign(tr.size() + 1, 0);
    for (size_t i = 0; i < tr.size(); ++i) stg[i + 1] = stg[i] + tr[i].len;
    if (by_dst) {
      order = dst_order(tr);
    } else {
      order.resize(tr.size());
      for (size_t i = 0; i < tr.size(); ++i) order[i] = int32_t(i);
    }
    for (const int32_t i : order) {
      const kvx_triple& t = tr[size_t(i)];
      for (int64_t o = 0; o < t.len; o += piece) {
        const int64_t len = std::min<int64_t>(piece, t.len - o);
        p->pieces.push_back(Piece{t.src_off + o, t.dst_off + o, stg[size_t(i)] + o, int32_t(len), r});
      }
    }
    p->payload[r] = stg.back();
  }
  if (p->nlists == 1) p->payload[1] = p->payload[0];
  if (!by_dst) {
    p->stream_pieces = p->pieces;
    std::sort(p->stream_pieces.begin(), p->stream_pieces.end(), [](const Piece& a, const Piece& b) {
      return a.reg != b.reg ? a.reg < b.reg : a.dst_off < b.dst_off;
    });
  }
}

}  // namespace

namespace kvx {

size_t worklist_bytes(const kvx_plan_t* p) {
  const size_t pb = p->pieces.size() * sizeof(Piece);
  const size_t sb = p->stream_pieces.size() * sizeof(Piece);
  const size_t bb = p->blocks.size() * sizeof(BlockPair);
  const size_t rb = p->runs_dst.size() * sizeof(RunRec);   // each of the two run tables
  const size_t gb = (p->gidx_dst.size() * sizeof(uint32_t) + 15) / 16 * 16;  // each run index, 16-B padded
  return std::max<size_t>(pb + sb + bb + 2 * rb + 2 * gb, 256);
}

int worklist_copy(kvx_plan_t* p, char* buf, hipStream_t s) {
  const size_t pb = p->pieces.size() * sizeof(Piece);
  const size_t sb = p->stream_pieces.size() * sizeof(Piece);
  const size_t bb = p->blocks.size() * sizeof(BlockPair);
  const size_t rb = p->runs_dst.size() * sizeof(RunRec);
  const size_t gb = (p->gidx_dst.size() * sizeof(uint32_t) + 15) / 16 * 16;
  hipError_t e;
  p->d_pieces = reinterpret_cast<const Piece*>(buf);
  p->d_stream = sb ? reinterpret_cast<const Piece*>(buf + pb) : p->d_pieces;
  p->d_blocks = reinterpret_cast<const BlockPair*>(buf + pb + sb);
  if (pb) {
    e = hipMemcpyAsync(buf, p->pieces.data(), pb, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(pieces)");
  }
  if (sb) {
    e = hipMemcpyAsync(buf + pb, p->stream_pieces.data(), sb, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(pieces)");
  }
  if (bb) {
    e = hipMemcpyAsync(buf + pb + sb, p->blocks.data(), bb, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(blocks)");
  }
  if (p->runs_mode) {
    char* const r0 = buf + pb + sb + bb;
    p->d_runs_dst = reinterpret_cast<const RunRec*>(r0);
    p->d_runs_plan = reinterpret_cast<const RunRec*>(r0 + rb);
    p->d_gidx_dst = reinterpret_cast<const uint32_t*>(r0 + 2 * rb);
    p->d_gidx_plan = reinterpret_cast<const uint32_t*>(r0 + 2 * rb + gb);
    const struct {
      const void* src;
      char* dst;
      size_t bytes;
    } parts[4] = {{p->runs_dst.data(), r0, rb},
                  {p->runs_plan.data(), r0 + rb, rb},
                  {p->gidx_dst.data(), r0 + 2 * rb, p->gidx_dst.size() * sizeof(uint32_t)},
                  {p->gidx_plan.data(), r0 + 2 * rb + gb, p->gidx_plan.size() * sizeof(uint32_t)}};
    for (const auto& part : parts) {
      if (!part.bytes) continue;
      e = hipMemcpyAsync(part.dst, part.src, part.bytes, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(run tables)");
    }
  }
  return KVX_OK;
}

}  // namespace kvx

namespace {

int upload(kvx_plan_t* p, hipStream_t s) {
  const size_t total = worklist_bytes(p);
  int rc = desc_alloc(total, &p->dev_buf, &p->device);
  if (rc != KVX_OK) {
    p->dev_buf = nullptr;
    return rc;
  }
  p->dev_bytes = total;
  rc = worklist_copy(p, static_cast<char*>(p->dev_buf), s);
  if (rc) return rc;
  hipError_t e = hipEventCreateWithFlags(&p->upload_ev, hipEventDisableTiming);
  if (e != hipSuccess) {
    p->upload_ev = nullptr;
    return fail_hip(e, "hipEventCreate(upload)");
  }
  e = hipEventRecord(p->upload_ev, s);
  if (e != hipSuccess) return fail_hip(e, "hipEventRecord(upload)");
  return KVX_OK;
}

// Free a plan.  Kernels may still be reading its descriptors on any stream,
// so the device is drained first (no per-launch bookkeeping is kept: a
// marker per launch would cost every push a queue packet).
void release(kvx_plan_t* p) {
  if (!p) return;
  if (p->dev_buf && !p->in_scratch) (void)hipDeviceSynchronize();
  kvx::plan_free_idle(p);
}

// Plans released with kvx_plan_destroy_after, each with the event recorded
// behind its last work; freed once the event has fired.
std::mutex g_retire_mu;
std::vector<std::pair<kvx_plan_t*, hipEvent_t>> g_retired;

// Free the retired plans whose event has fired (wait: wait for each).
// *pending receives how many remain.
int reclaim(bool wait, int64_t* pending) {
  std::lock_guard<std::mutex> lk(g_retire_mu);
  int rc = KVX_OK;
  for (size_t i = 0; i < g_retired.size();) {
    const hipEvent_t ev = g_retired[i].second;
    const hipError_t e = wait ? hipEventSynchronize(ev) : hipEventQuery(ev);
    if (e == hipSuccess) {
      (void)hipEventDestroy(ev);
      kvx::plan_free_idle(g_retired[i].first);
      g_retired[i] = g_retired.back();
      g_retired.pop_back();
      continue;
    }
    if (e != hipErrorNotReady && rc == KVX_OK) rc = fail_hip(e, "kvx_plan_reclaim: event");
    ++i;
  }
  if (pending && rc == KVX_OK) *pending = int64_t(g_retired.size());
  return rc;
}

// First token a sliding-window group moves ([MORI] §6: sliding-window layers
// get their own geometry).  The receiving side's next query, at position n,
// sees positions n-W+1 .. n; blocks holding none of them are skipped, so the
// move starts at the later of the two sides' starts of the block holding
// position n-W+1.
int64_t window_first(int64_t n, int32_t w, int64_t bss, int64_t bsd) {
  if (w <= 0) return 0;
  const int64_t first = std::max<int64_t>(0, n - w + 1);
  return std::max(first / bss * bss, first / bsd * bsd);
}

// Validate the requests and build the plan's block list, runs and triples.
// Validation order per request: token count, both list lengths, source IDs,
// then destination IDs (range, then reuse across the plan).  With a sliding
// window, the entries of skipped blocks are not looked at.
int build_plan(kvx_plan_t* p, int32_t R, const int64_t* num_tokens, const int64_t* so,
               const int64_t* dof, const int32_t* src_ids, const int32_t* dst_ids) {
  const Geom& gs = p->src;
  const Geom& gd = p->dst;
  const int64_t bss = gs.BS, bsd = gd.BS;
  if (R > 0 && (so[0] < 0 || dof[0] < 0)) return fail(KVX_E_INVAL, "kvx_plan: negative first offset");
  // Each planned block takes one source ID of the caller's lists, so their
  // total length bounds the block list.  Nothing is validated yet, so the
  // reservation is capped (4M blocks, 64 MiB); past that the list grows.
  if (bss == bsd && R > 0 && so[R] > so[0]) {
    const size_t cap = size_t(std::min<int64_t>(so[R] - so[0], int64_t(1) << 22));
    p->blocks.reserve(cap);
    p->runs.reserve(cap);
  }
  std::vector<uint8_t> dst_used(size_t(gd.NB), 0);
  for (int32_t r = 0; r < R; ++r) {
    const int64_t n = num_tokens[r];
    if (n < 0) return fail(KVX_E_INVAL, "kvx_plan: request %d: negative token count", r);
    if (so[r + 1] < so[r] || dof[r + 1] < dof[r])
      return fail(KVX_E_INVAL, "kvx_plan: offsets not monotone at request %d", r);
    const int64_t nbs = (n + bss - 1) / bss, nbd = (n + bsd - 1) / bsd;
    if (so[r + 1] - so[r] < nbs || dof[r + 1] - dof[r] < nbd)
      return fail(KVX_E_INVAL, "kvx_plan: request %d: block list shorter than its %lld/%lld blocks", r,
                  (long long)nbs, (long long)nbd);
    if (n == 0) continue;
    if (!src_ids || !dst_ids) return fail(KVX_E_INVAL, "kvx_plan: null block ID array");
    const int32_t* S = src_ids + so[r];
    const int32_t* Dd = dst_ids + dof[r];
    const int64_t t0 = window_first(n, gs.window, bss, bsd);
    const int64_t js = t0 / bss;
    for (int64_t i = js; i < nbs; ++i)
      if (S[i] < 0 || S[i] >= gs.NB)
        return fail(KVX_E_RANGE, "kvx_plan: request %d: src block %d outside [0,%d)", r, S[i], gs.NB);
    for (int64_t i = t0 / bsd; i < nbd; ++i) {
      if (Dd[i] < 0 || Dd[i] >= gd.NB)
        return fail(KVX_E_RANGE, "kvx_plan: request %d: dst block %d outside [0,%d)", r, Dd[i], gd.NB);
      if (dst_used[size_t(Dd[i])]) return fail(KVX_E_DUPDST, "kvx_plan: dst block %d used twice", Dd[i]);
      dst_used[size_t(Dd[i])] = 1;
    }
    if (t0 >= n) continue;
    if (bss == bsd) {
      // Merge ([PUSH] "Threading-Modell"; [MORI] §3.1, §6): a new run starts
      // at the request's first moved block and wherever either side is not
      // the previous block + 1.
      const int32_t tail = int32_t(n - (nbs - 1) * bss);
      int64_t start = js;
      for (int64_t i = js + 1; i <= nbs; ++i) {
        if (i == nbs || S[i] != S[i - 1] + 1 || Dd[i] != Dd[i - 1] + 1) {
          p->runs.push_back(kvx_run{S[start], Dd[start], int32_t(i - start), i == nbs ? tail : int32_t(bss)});
          start = i;
        }
      }
      for (int64_t i = js; i < nbs; ++i)
        p->blocks.push_back(BlockPair{S[i], Dd[i], i == nbs - 1 ? tail : int32_t(bss), 0});
    } else {
      // Different block sizes ([PUSH] "Implementierungsdetails" step 3):
      // token t sits in source block S[t / BSs], slot t % BSs and lands in
      // destination block Dd[t / BSd], slot t % BSd.  Cut the token range
      // wherever either side enters a new block.
      for (int64_t t = t0; t < n;) {
        const int64_t ss = t % bss, ds = t % bsd;
        const int64_t k = std::min({bss - ss, bsd - ds, n - t});
        p->blocks.push_back(BlockPair{S[t / bss], Dd[t / bsd], int32_t(k), pack_slots(ss, ds)});
        t += k;
      }
    }
  }
  if (p->push_ok) {
    build_triples(p);
    build_pieces(p);
  } else {
    // Pools that differ in head count or layout only take kvx_copy_heads,
    // which moves each planned block on its own: the block order is not
    // observable, and in source order its strided reads run 1-3% faster (the
    // TP4 head share, side by side on two boxes; destination order changed
    // nothing).
    std::sort(p->blocks.begin(), p->blocks.end(), [](const BlockPair& a, const BlockPair& b) {
      if (a.src != b.src) return a.src < b.src;
      return a.dst != b.dst ? a.dst < b.dst : a.slots < b.slots;
    });
  }
  p->scale_seg_bytes = gs.scales ? pad16(4 * int64_t(p->blocks.size())) : 0;
  return KVX_OK;
}

// State-slot plan ([MORI] §6: the conv and SSM regions move slot by slot).
// A request moving at least one token moves the slot its list starts with;
// each one is a run, and each region's triples merge neighbouring slots.
int build_state_plan(kvx_plan_t* p, int32_t R, const int64_t* num_tokens, const int64_t* so,
                     const int64_t* dof, const int32_t* src_ids, const int32_t* dst_ids) {
  const Geom& gs = p->src;
  const Geom& gd = p->dst;
  if (R > 0 && (so[0] < 0 || dof[0] < 0)) return fail(KVX_E_INVAL, "kvx_plan: negative first offset");
  std::vector<uint8_t> dst_used(size_t(gd.NB), 0);
  for (int32_t r = 0; r < R; ++r) {
    const int64_t n = num_tokens[r];
    if (n < 0) return fail(KVX_E_INVAL, "kvx_plan: request %d: negative token count", r);
    if (so[r + 1] < so[r] || dof[r + 1] < dof[r])
      return fail(KVX_E_INVAL, "kvx_plan: offsets not monotone at request %d", r);
    if (n == 0) continue;
    if (so[r + 1] - so[r] < 1 || dof[r + 1] - dof[r] < 1)
      return fail(KVX_E_INVAL, "kvx_plan: request %d: no state slot", r);
    if (!src_ids || !dst_ids) return fail(KVX_E_INVAL, "kvx_plan: null slot ID array");
    const int32_t s = src_ids[so[r]], d = dst_ids[dof[r]];
    if (s < 0 || s >= gs.NB)
      return fail(KVX_E_RANGE, "kvx_plan: request %d: src slot %d outside [0,%d)", r, s, gs.NB);
    if (d < 0 || d >= gd.NB)
      return fail(KVX_E_RANGE, "kvx_plan: request %d: dst slot %d outside [0,%d)", r, d, gd.NB);
    if (dst_used[size_t(d)]) return fail(KVX_E_DUPDST, "kvx_plan: dst slot %d used twice", d);
    dst_used[size_t(d)] = 1;
    p->runs.push_back(kvx_run{s, d, 1, 1});
    for (int reg = 0; reg < 2; ++reg) {
      const int64_t sb = gs.slot_bytes[reg];
      emit(p->triples[reg], int64_t(s) * sb, int64_t(d) * sb, sb);
    }
  }
  build_pieces(p);
  return KVX_OK;
}

}  // namespace

extern "C" {

int kvx_plan(const kvx_pool* src, const kvx_pool* dst, int32_t num_requests,
             const int64_t* num_tokens, const int64_t* src_offsets, const int64_t* dst_offsets,
             const int32_t* src_ids, const int32_t* dst_ids, uint32_t flags, hipStream_t upload_stream,
             kvx_plan_t** out) {
  if (!src || !dst || !out) return fail(KVX_E_INVAL, "kvx_plan: null pool or output");
  if (!(flags & KVX_PLAN_HOST_ONLY)) (void)reclaim(false, nullptr);  // plans released earlier whose work is done
  kvx_plan_t* p = nullptr;
  int rc = kvx::plan_build(src, dst, num_requests, num_tokens, src_offsets, dst_offsets, src_ids, dst_ids, flags,
                           upload_stream, &p);
  if (rc) return rc;
  if (!p->host_only) rc = upload(p, upload_stream);
  if (rc != KVX_OK) {
    release(p);
    return rc;
  }
  *out = p;
  return KVX_OK;
}

}  // extern "C"

int kvx::plan_build(const kvx_pool* src, const kvx_pool* dst, int32_t num_requests, const int64_t* num_tokens,
                    const int64_t* src_offsets, const int64_t* dst_offsets, const int32_t* src_ids,
                    const int32_t* dst_ids, uint32_t flags, hipStream_t upload_stream, kvx_plan_t** out) {
  if (!src || !dst || !out) return fail(KVX_E_INVAL, "kvx_plan: null pool or output");
  if (src == dst) return fail(KVX_E_INVAL, "kvx_plan: src and dst are the same pool");
  if (flags & ~(KVX_PLAN_HOST_ONLY | KVX_PLAN_OVERLAP | KVX_PLAN_RUNS))
    return fail(KVX_E_INVAL, "kvx_plan: unknown flags 0x%x", flags);
  if (!(flags & KVX_PLAN_HOST_ONLY) && capturing(upload_stream))
    return fail(KVX_E_INVAL, "kvx_plan: the upload stream is capturing a graph (build plans outside a capture)");
  if (num_requests < 0) return fail(KVX_E_INVAL, "kvx_plan: negative request count");
  if (num_requests > 0 && (!num_tokens || !src_offsets || !dst_offsets))
    return fail(KVX_E_INVAL, "kvx_plan: null num_tokens or offsets");
  const Geom& gs = src->g;
  const Geom& gd = dst->g;
  if (gs.state != gd.state) return fail(KVX_E_MISMATCH, "kvx_plan: one pool holds state slots, the other KV");
  if (gs.state) {
    if (gs.L != gd.L || gs.slot_bytes[0] != gd.slot_bytes[0] || gs.slot_bytes[1] != gd.slot_bytes[1])
      return fail(KVX_E_MISMATCH, "kvx_plan: state pools differ in layers or slot sizes");
  } else {
    if (gs.L != gd.L || gs.D != gd.D || gs.E != gd.E || gs.scales != gd.scales || gs.nreg != gd.nreg)
      return fail(KVX_E_MISMATCH, "kvx_plan: pools differ in layers/head_dim/elem_bytes/scales/regions");
    if (gs.window != gd.window)
      return fail(KVX_E_MISMATCH, "kvx_plan: sliding windows differ (%d vs %d)", gs.window, gd.window);
    if (gs.BS != gd.BS && gs.scales)
      return fail(KVX_E_UNSUPPORTED, "kvx_plan: per-block scales need equal block sizes (%d vs %d)", gs.BS, gd.BS);
  }

  kvx_plan_t* p = new (std::nothrow) kvx_plan_t;
  if (!p) return fail(KVX_E_NOMEM, "kvx_plan: out of host memory");
  int rc = KVX_OK;
  try {
    p->src = gs;
    p->dst = gd;
    p->push_ok = gs.state || (gs.H == gd.H && gs.layout == gd.layout);
    p->host_only = (flags & KVX_PLAN_HOST_ONLY) != 0;
    p->overlap = (flags & KVX_PLAN_OVERLAP) != 0;
    p->want_runs = (flags & KVX_PLAN_RUNS) != 0;
    p->nreg = gs.nreg;
    p->nlists = gs.state ? 2 : 1;
    rc = gs.state ? build_state_plan(p, num_requests, num_tokens, src_offsets, dst_offsets, src_ids, dst_ids)
                  : build_plan(p, num_requests, num_tokens, src_offsets, dst_offsets, src_ids, dst_ids);
  } catch (const std::bad_alloc&) {
    rc = fail(KVX_E_NOMEM, "kvx_plan: out of host memory");
  }
  if (rc != KVX_OK) {
    release(p);
    return rc;
  }
  *out = p;
  return KVX_OK;
}

extern "C" {

int kvx_plan_runs(const kvx_plan_t* p, kvx_run* out, int64_t cap, int64_t* n) {
  if (!p || !n) return fail(KVX_E_INVAL, "kvx_plan_runs: null argument");
  if (!p->src.state && p->src.BS != p->dst.BS)
    return fail(KVX_E_MISMATCH, "kvx_plan_runs: block runs need equal block sizes (%d vs %d)", p->src.BS, p->dst.BS);
  const int64_t cnt = int64_t(p->runs.size());
  if (out && cap >= cnt) std::copy(p->runs.begin(), p->runs.end(), out);
  *n = cnt;
  return KVX_OK;
}

int kvx_plan_triples(const kvx_plan_t* p, int32_t layer, int32_t kv, kvx_triple* out, int64_t cap,
                     int64_t* n) {
  if (!p || !n) return fail(KVX_E_INVAL, "kvx_plan_triples: null argument");
  if (layer < 0 || layer >= p->src.L || kv < 0 || kv >= p->nreg)
    return fail(KVX_E_RANGE, "kvx_plan_triples: layer %d / region %d out of range", layer, kv);
  if (!p->push_ok)
    return fail(KVX_E_MISMATCH, "kvx_plan_triples: pools differ in head count or layout");
  const std::vector<kvx_triple>& t = p->region_triples(kv);
  const int64_t cnt = int64_t(t.size());
  if (out && cap >= cnt) std::copy(t.begin(), t.end(), out);
  *n = cnt;
  return KVX_OK;
}

int kvx_plan_wait(const kvx_plan_t* cp) {
  if (!cp) return fail(KVX_E_INVAL, "kvx_plan_wait: null plan");
  kvx_plan_t* p = const_cast<kvx_plan_t*>(cp);
  if (p->host_only || p->upload_seen.load(std::memory_order_acquire)) return KVX_OK;
  const hipError_t e = hipEventSynchronize(p->upload_ev);
  if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize(upload)");
  p->upload_seen.store(true, std::memory_order_release);
  return KVX_OK;
}

int kvx_plan_bytes(const kvx_plan_t* p, int64_t* rd, int64_t* wr) {
  if (!p || !rd || !wr) return fail(KVX_E_INVAL, "kvx_plan_bytes: null argument");
  if (!p->push_ok) return fail(KVX_E_MISMATCH, "kvx_plan_bytes: pools differ in head count or layout");
  const int64_t sc = p->src.scales ? 4 * int64_t(p->blocks.size()) : 0;
  int64_t b = 0;
  for (int r = 0; r < p->nreg; ++r) b += p->payload[r] + sc;
  *rd = b;
  *wr = b;
  return KVX_OK;
}

int kvx_plan_launch_shape(const kvx_plan_t* p, kvx_launch_shape* out) {
  if (!p || !out) return fail(KVX_E_INVAL, "kvx_plan_launch_shape: null argument");
  if (!p->push_ok) return fail(KVX_E_MISMATCH, "kvx_plan_launch_shape: pools differ in head count or layout");
  out->pieces = p->runs_mode ? (int64_t(p->run_total16) + kRunChunk16 - 1) / kRunChunk16 * p->nreg
                             : int64_t(p->pieces.size()) * (p->nlists == 1 ? p->nreg : 1);
  out->piece_bytes = int32_t(shape_piece_bytes(p->shape));
  out->lanes = kShapes[p->shape].threads;
  out->vectors = kShapes[p->shape].vecs;
  out->run_table = p->runs_mode ? 1 : 0;
  return KVX_OK;
}

void kvx_plan_destroy(kvx_plan_t* p) { release(p); }

int kvx_plan_destroy_after(kvx_plan_t* p, hipStream_t stream) {
  if (!p) return KVX_OK;
  if (!p->dev_buf || p->in_scratch) {  // host-only, or a work list the library never frees
    plan_free_idle(p);
    return KVX_OK;
  }
  if (capturing(stream)) return fail(KVX_E_INVAL, "kvx_plan_destroy_after: the stream is capturing a graph");
  hipEvent_t ev = nullptr;
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e != hipSuccess) return fail_hip(e, "kvx_plan_destroy_after: hipEventCreate");
  e = hipEventRecord(ev, stream);
  if (e != hipSuccess) {
    (void)hipEventDestroy(ev);
    return fail_hip(e, "kvx_plan_destroy_after: hipEventRecord");
  }
  try {
    std::lock_guard<std::mutex> lk(g_retire_mu);
    g_retired.emplace_back(p, ev);
  } catch (const std::bad_alloc&) {
    (void)hipEventDestroy(ev);
    return fail(KVX_E_NOMEM, "kvx_plan_destroy_after: out of host memory");
  }
  return reclaim(false, nullptr);
}

int kvx_plan_reclaim(int32_t wait, int64_t* pending) { return reclaim(wait != 0, pending); }

int kvx_staging_bytes(const kvx_plan_t* p, int32_t l0, int32_t l1, int64_t* bytes) {
  if (!p || !bytes) return fail(KVX_E_INVAL, "kvx_staging_bytes: null argument");
  if (l0 < 0 || l1 < l0 || l1 > p->src.L)
    return fail(KVX_E_RANGE, "kvx_staging_bytes: layers [%d,%d) outside [0,%d]", l0, l1, p->src.L);
  if (!p->push_ok) return fail(KVX_E_MISMATCH, "kvx_staging_bytes: pools differ in head count or layout");
  *bytes = int64_t(l1 - l0) * p->stg_layer();
  return KVX_OK;
}

}  // extern "C"
