/* A C99 consumer of the libkvx device calls: two K/V pools in device memory,
 * a plan for three requests, then kvx_push_layer for every layer,
 * kvx_pack + kvx_unpack over all layers, one kvx_push_many call, and every
 * layer through a stream's write queue behind events of another stream, each
 * checked byte for byte on the host against the per-token definition: token
 * t of a request that moves n tokens (prompt - computed - 1, [MORI] §3.1)
 * goes from slot t % BS of source block src[t / BS] to slot t % BS of
 * destination block dst[t / BS], in every layer and in both regions (NHD rows
 * of H*D*E bytes).  The staging buffer is the moved token rows in (layer,
 * region, request, token) order.  Last, one TP rank's head slice: source
 * head 1 of every moved token lands as head 0 of a one-head HND pool
 * ([blk][head][slot][d]) through kvx_copy_heads_layers, and again layer by
 * layer through a write queue.  Prints "ok" and exits 0 when every check
 * holds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvx.h"

enum { L = 3, NB = 96, BS = 16, H = 2, D = 64, E = 2, R = 3 };
#define TOKEN_BYTES ((size_t)H * D * E)
#define BLOCK_BYTES ((size_t)BS * TOKEN_BYTES)
#define REGION_BYTES ((size_t)NB * BLOCK_BYTES)
#define POOL_BYTES ((size_t)L * 2 * REGION_BYTES)
/* the one-head HND pool of the head-slice check */
#define HEAD_BYTES ((size_t)D * E)
#define HBLOCK_BYTES ((size_t)BS * HEAD_BYTES)
#define HREGION_BYTES ((size_t)NB * HBLOCK_BYTES)
#define HPOOL_BYTES ((size_t)L * 2 * HREGION_BYTES)

static int failures = 0;

#define HIP_OK(call)                                                         \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s failed at line %d: %d\n", #call, __LINE__, (int)e_); \
      exit(1);                                                               \
    }                                                                        \
  } while (0)

#define KVX_OK_(call)                                                                  \
  do {                                                                                 \
    int s_ = (call);                                                                   \
    if (s_ != KVX_OK) {                                                                \
      fprintf(stderr, "%s failed at line %d: %s (%s)\n", #call, __LINE__, kvx_status_str(s_), \
              kvx_last_error());                                                       \
      exit(1);                                                                         \
    }                                                                                  \
  } while (0)

static size_t region_off(int layer, int reg) { return ((size_t)layer * 2 + (size_t)reg) * REGION_BYTES; }

static kvx_pool* make_pool_of(uint8_t* base, size_t region_bytes, int32_t heads, int32_t layout) {
  void* kb[L];
  void* vb[L];
  kvx_pool_desc d;
  kvx_pool* p = NULL;
  int l;
  for (l = 0; l < L; ++l) {
    kb[l] = base + ((size_t)l * 2 + 0) * region_bytes;
    vb[l] = base + ((size_t)l * 2 + 1) * region_bytes;
  }
  memset(&d, 0, sizeof d);
  d.num_layers = L;
  d.num_blocks = NB;
  d.block_size = BS;
  d.num_heads = heads;
  d.head_dim = D;
  d.elem_bytes = E;
  d.layout = layout;
  d.k_base = kb;
  d.v_base = vb;
  KVX_OK_(kvx_pool_create(&d, &p));
  return p;
}

static kvx_pool* make_pool(uint8_t* base) { return make_pool_of(base, REGION_BYTES, H, KVX_NHD); }

/* The expected destination pool: `init` with every moved token row copied. */
static void expect(const uint8_t* src, const uint8_t* init, uint8_t* out, const int64_t* n, const int64_t* so,
                   const int32_t* sid, const int32_t* did) {
  int l, reg, r;
  int64_t t;
  memcpy(out, init, POOL_BYTES);
  for (l = 0; l < L; ++l)
    for (reg = 0; reg < 2; ++reg)
      for (r = 0; r < R; ++r)
        for (t = 0; t < n[r]; ++t) {
          const size_t slot = (size_t)(t % BS) * TOKEN_BYTES;
          const size_t s = region_off(l, reg) + (size_t)sid[so[r] + t / BS] * BLOCK_BYTES + slot;
          const size_t d = region_off(l, reg) + (size_t)did[so[r] + t / BS] * BLOCK_BYTES + slot;
          memcpy(out + d, src + s, TOKEN_BYTES);
        }
}

static void check_pool(const char* what, uint8_t* dev, const uint8_t* want, uint8_t* scratch) {
  HIP_OK(hipMemcpy(scratch, dev, POOL_BYTES, hipMemcpyDeviceToHost));
  if (memcmp(scratch, want, POOL_BYTES) != 0) {
    fprintf(stderr, "%s: destination pool differs from the per-token definition\n", what);
    ++failures;
  }
}

int main(void) {
  /* prompts of 70, 33 and 17 tokens: 69 (ragged tail), 32 and 16 tokens move */
  const int64_t prompts[R] = {70, 33, 17};
  /* one CSR offset array serves both sides: each request lists as many
   * source as destination blocks */
  const int64_t off[R + 1] = {0, 5, 7, 8};
  const int32_t src_ids[8] = {5, 6, 7, 8, 40, 9, 10, 60};
  const int32_t dst_ids[8] = {70, 71, 20, 21, 22, 11, 12, 95};
  int64_t n[R];
  uint8_t *h_src, *h_init, *h_want, *h_got, *h_stg, *h_stg_want;
  uint8_t *d_src, *d_dst, *d_stg;
  kvx_pool *ps, *pd;
  kvx_plan_t* plan = NULL;
  const kvx_plan_t* plans[L];
  int32_t layers[L];
  hipStream_t s;
  int64_t nstg = 0;
  size_t i, pos;
  int l, reg, r;
  int64_t t;

  for (r = 0; r < R; ++r) n[r] = kvx_tokens_to_move(prompts[r], 0);
  h_src = malloc(POOL_BYTES);
  h_init = malloc(POOL_BYTES);
  h_want = malloc(POOL_BYTES);
  h_got = malloc(POOL_BYTES);
  if (!h_src || !h_init || !h_want || !h_got) return 1;
  for (i = 0; i < POOL_BYTES; ++i) {
    h_src[i] = (uint8_t)((i * 2654435761u) >> 13);
    h_init[i] = (uint8_t)(0xa5 ^ (i >> 7));
  }
  HIP_OK(hipStreamCreate(&s));
  HIP_OK(hipMalloc((void**)&d_src, POOL_BYTES));
  HIP_OK(hipMalloc((void**)&d_dst, POOL_BYTES));
  HIP_OK(hipMemcpy(d_src, h_src, POOL_BYTES, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_dst, h_init, POOL_BYTES, hipMemcpyHostToDevice));
  ps = make_pool(d_src);
  pd = make_pool(d_dst);
  KVX_OK_(kvx_plan(ps, pd, R, n, off, off, src_ids, dst_ids, 0u, s, &plan));
  expect(h_src, h_init, h_want, n, off, src_ids, dst_ids);

  /* layer by layer */
  for (l = 0; l < L; ++l) KVX_OK_(kvx_push_layer(plan, l, NULL, s));
  HIP_OK(hipStreamSynchronize(s));
  check_pool("kvx_push_layer", d_dst, h_want, h_got);

  /* staging round trip into a reset destination */
  KVX_OK_(kvx_staging_bytes(plan, 0, L, &nstg));
  if (nstg != (int64_t)L * 2 * (n[0] + n[1] + n[2]) * (int64_t)TOKEN_BYTES) {
    fprintf(stderr, "staging bytes %lld\n", (long long)nstg);
    ++failures;
  }
  h_stg = malloc((size_t)nstg);
  h_stg_want = malloc((size_t)nstg);
  if (!h_stg || !h_stg_want) return 1;
  pos = 0;
  for (l = 0; l < L; ++l)
    for (reg = 0; reg < 2; ++reg)
      for (r = 0; r < R; ++r)
        for (t = 0; t < n[r]; ++t) {
          const size_t sidx = region_off(l, reg) + (size_t)src_ids[off[r] + t / BS] * BLOCK_BYTES +
                              (size_t)(t % BS) * TOKEN_BYTES;
          memcpy(h_stg_want + pos, h_src + sidx, TOKEN_BYTES);
          pos += TOKEN_BYTES;
        }
  HIP_OK(hipMalloc((void**)&d_stg, (size_t)nstg));
  HIP_OK(hipMemcpy(d_dst, h_init, POOL_BYTES, hipMemcpyHostToDevice));
  KVX_OK_(kvx_pack(plan, 0, L, d_stg, nstg, s));
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(h_stg, d_stg, (size_t)nstg, hipMemcpyDeviceToHost));
  if (memcmp(h_stg, h_stg_want, (size_t)nstg) != 0) {
    fprintf(stderr, "kvx_pack: staging differs from the moved rows in order\n");
    ++failures;
  }
  KVX_OK_(kvx_unpack(plan, 0, L, d_stg, nstg, s));
  HIP_OK(hipStreamSynchronize(s));
  check_pool("kvx_unpack", d_dst, h_want, h_got);

  /* every layer in one kvx_push_many call */
  HIP_OK(hipMemcpy(d_dst, h_init, POOL_BYTES, hipMemcpyHostToDevice));
  for (l = 0; l < L; ++l) {
    plans[l] = plan;
    layers[l] = l;
  }
  KVX_OK_(kvx_push_many(plans, layers, L, NULL, s));
  HIP_OK(hipStreamSynchronize(s));
  check_pool("kvx_push_many", d_dst, h_want, h_got);

  /* every layer through the write queue of `s`, each behind an event that
   * another stream records after a copy of its own */
  {
    hipStream_t c;
    hipEvent_t ev[L], done;
    kvx_queue* q = NULL;
    uint8_t* d_busy;
    int64_t writes = 0, groups = 0, launches = 0;
    HIP_OK(hipStreamCreate(&c));
    HIP_OK(hipMalloc((void**)&d_busy, POOL_BYTES));
    for (l = 0; l < L; ++l) HIP_OK(hipEventCreateWithFlags(&ev[l], hipEventDisableTiming));
    HIP_OK(hipEventCreateWithFlags(&done, hipEventDisableTiming));
    HIP_OK(hipMemcpy(d_dst, h_init, POOL_BYTES, hipMemcpyHostToDevice));
    KVX_OK_(kvx_queue_create(s, &q));
    for (l = 0; l < L; ++l) {
      HIP_OK(hipMemcpyAsync(d_busy, d_src, POOL_BYTES, hipMemcpyDeviceToDevice, c));
      HIP_OK(hipEventRecord(ev[l], c));
      KVX_OK_(kvx_queue_push(q, plan, l, ev[l]));
    }
    KVX_OK_(kvx_queue_flush(q));
    HIP_OK(hipEventRecord(done, s));
    HIP_OK(hipEventSynchronize(done));
    check_pool("kvx_queue", d_dst, h_want, h_got);
    KVX_OK_(kvx_queue_stats(q, &writes, &groups, &launches));
    if (writes != L || groups < 1 || groups > L || launches < groups) {
      fprintf(stderr, "kvx_queue_stats: %lld writes, %lld groups, %lld launches\n", (long long)writes,
              (long long)groups, (long long)launches);
      ++failures;
    }
    KVX_OK_(kvx_queue_destroy(q));
    HIP_OK(hipStreamSynchronize(c));
    for (l = 0; l < L; ++l) HIP_OK(hipEventDestroy(ev[l]));
    HIP_OK(hipEventDestroy(done));
    HIP_OK(hipFree(d_busy));
    HIP_OK(hipStreamDestroy(c));
  }

  /* head 1 of every moved token row into head 0 of a one-head HND pool */
  {
    uint8_t *d_h, *h_hinit, *h_hwant, *h_hgot;
    kvx_pool* ph;
    kvx_plan_t* hplan = NULL;
    h_hinit = malloc(HPOOL_BYTES);
    h_hwant = malloc(HPOOL_BYTES);
    h_hgot = malloc(HPOOL_BYTES);
    if (!h_hinit || !h_hwant || !h_hgot) return 1;
    for (i = 0; i < HPOOL_BYTES; ++i) h_hinit[i] = (uint8_t)(0x3c ^ (i >> 5));
    memcpy(h_hwant, h_hinit, HPOOL_BYTES);
    for (l = 0; l < L; ++l)
      for (reg = 0; reg < 2; ++reg)
        for (r = 0; r < R; ++r)
          for (t = 0; t < n[r]; ++t) {
            const size_t sidx = region_off(l, reg) + (size_t)src_ids[off[r] + t / BS] * BLOCK_BYTES +
                                (size_t)(t % BS) * TOKEN_BYTES + 1 * HEAD_BYTES;
            const size_t didx = ((size_t)l * 2 + (size_t)reg) * HREGION_BYTES +
                                (size_t)dst_ids[off[r] + t / BS] * HBLOCK_BYTES + (size_t)(t % BS) * HEAD_BYTES;
            memcpy(h_hwant + didx, h_src + sidx, HEAD_BYTES);
          }
    HIP_OK(hipMalloc((void**)&d_h, HPOOL_BYTES));
    HIP_OK(hipMemcpy(d_h, h_hinit, HPOOL_BYTES, hipMemcpyHostToDevice));
    ph = make_pool_of(d_h, HREGION_BYTES, 1, KVX_HND);
    KVX_OK_(kvx_plan(ps, ph, R, n, off, off, src_ids, dst_ids, 0u, s, &hplan));
    KVX_OK_(kvx_copy_heads_layers(hplan, 0, L, 1, 0, 1, NULL, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(h_hgot, d_h, HPOOL_BYTES, hipMemcpyDeviceToHost));
    if (memcmp(h_hgot, h_hwant, HPOOL_BYTES) != 0) {
      fprintf(stderr, "kvx_copy_heads_layers: head-slice pool differs from the per-token definition\n");
      ++failures;
    }
    /* the same slice layer by layer through a write queue */
    {
      kvx_queue* hq = NULL;
      hipEvent_t hdone;
      HIP_OK(hipMemcpy(d_h, h_hinit, HPOOL_BYTES, hipMemcpyHostToDevice));
      HIP_OK(hipEventCreateWithFlags(&hdone, hipEventDisableTiming));
      KVX_OK_(kvx_queue_create(s, &hq));
      for (l = 0; l < L; ++l) KVX_OK_(kvx_queue_push_heads(hq, hplan, l, 1, 0, 1, NULL));
      KVX_OK_(kvx_queue_flush(hq));
      HIP_OK(hipEventRecord(hdone, s));
      HIP_OK(hipEventSynchronize(hdone));
      HIP_OK(hipMemcpy(h_hgot, d_h, HPOOL_BYTES, hipMemcpyDeviceToHost));
      if (memcmp(h_hgot, h_hwant, HPOOL_BYTES) != 0) {
        fprintf(stderr, "kvx_queue_push_heads: head-slice pool differs from the per-token definition\n");
        ++failures;
      }
      if (kvx_queue_push_heads(hq, hplan, 0, 0, 0, 2, NULL) != KVX_E_RANGE) {
        fprintf(stderr, "a queued two-head slice of a one-head pool was not refused\n");
        ++failures;
      }
      KVX_OK_(kvx_queue_destroy(hq));
      HIP_OK(hipEventDestroy(hdone));
    }
    /* a slice past the destination's one head is refused */
    if (kvx_copy_heads(hplan, 0, 0, 0, 2, NULL, s) != KVX_E_RANGE) {
      fprintf(stderr, "a two-head slice of a one-head pool was not refused\n");
      ++failures;
    }
    kvx_plan_destroy(hplan);
    kvx_pool_destroy(ph);
    HIP_OK(hipFree(d_h));
    free(h_hinit);
    free(h_hwant);
    free(h_hgot);
  }

  /* an out-of-range layer is refused and enqueues nothing */
  if (kvx_push_layer(plan, L, NULL, s) != KVX_E_RANGE) {
    fprintf(stderr, "layer %d was not refused\n", L);
    ++failures;
  }

  kvx_plan_destroy(plan);
  kvx_pool_destroy(ps);
  kvx_pool_destroy(pd);
  HIP_OK(hipFree(d_stg));
  HIP_OK(hipFree(d_src));
  HIP_OK(hipFree(d_dst));
  HIP_OK(hipStreamDestroy(s));
  free(h_src);
  free(h_init);
  free(h_want);
  free(h_got);
  free(h_stg);
  free(h_stg_want);
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
