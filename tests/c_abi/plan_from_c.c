/* A C99 consumer of the libkvx ABI: the header compiles as C, and a
 * host-only plan built through it has the runs, triples and byte counts the
 * run-merge definition gives for a small case worked by hand ([MORI] §3.1
 * and §6: prompt - computed - 1 tokens move; blocks consecutive on both
 * sides merge into one run; each run is one contiguous byte range per
 * (layer, region) in NHD).  Host-only plans never dereference the pool
 * addresses, so made-up 16-byte-aligned ones are registered.  Prints "ok"
 * and exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvx.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

enum { L = 2, NB = 64, BS = 16, H = 2, D = 64, E = 2 };
#define TOKEN_BYTES ((int64_t)H * D * E) /* 256 */
#define BLOCK_BYTES (BS * TOKEN_BYTES)   /* 4096 */
#define REGION_BYTES (NB * BLOCK_BYTES)

static kvx_pool* make_pool(uintptr_t base) {
  void* kb[L];
  void* vb[L];
  kvx_pool_desc d;
  kvx_pool* p = NULL;
  int l;
  for (l = 0; l < L; ++l) {
    kb[l] = (void*)(base + (uintptr_t)(2 * l) * REGION_BYTES);
    vb[l] = (void*)(base + (uintptr_t)(2 * l + 1) * REGION_BYTES);
  }
  memset(&d, 0, sizeof d);
  d.num_layers = L;
  d.num_blocks = NB;
  d.block_size = BS;
  d.num_heads = H;
  d.head_dim = D;
  d.elem_bytes = E;
  d.layout = KVX_NHD;
  d.k_base = kb;
  d.v_base = vb;
  CHECK(kvx_pool_create(&d, &p) == KVX_OK);
  return p;
}

int main(void) {
  kvx_pool* src;
  kvx_pool* dst;
  kvx_plan_t* plan = NULL;
  kvx_plan_t* bad = NULL;
  kvx_run runs[4];
  kvx_triple trip[4];
  int64_t n = 0, rd = 0, wr = 0, stg = 0;
  const int64_t offsets[2] = {0, 3};
  const int32_t src_ids[3] = {3, 4, 5};
  const int32_t dst_ids[3] = {10, 11, 20};
  const int32_t dup_ids[3] = {10, 11, 10};
  const int32_t far_ids[3] = {3, 4, NB};
  int64_t tokens;

  CHECK(kvx_abi_version() == KVX_ABI_VERSION);
  tokens = kvx_tokens_to_move(41, 0); /* the consumer recomputes the last prompt token */
  CHECK(tokens == 40);
  CHECK(kvx_should_reuse(512, 512) == 1 && kvx_should_reuse(511, 512) == 0);

  src = make_pool((uintptr_t)1 << 40);
  dst = make_pool((uintptr_t)1 << 41);
  CHECK(kvx_plan(src, dst, 1, &tokens, offsets, offsets, src_ids, dst_ids, KVX_PLAN_HOST_ONLY, NULL, &plan) ==
        KVX_OK);

  /* 40 tokens in 3 blocks, the last holding 8; 3,4 -> 10,11 merge, 5 -> 20 does not */
  CHECK(kvx_plan_runs(plan, NULL, 0, &n) == KVX_OK && n == 2);
  CHECK(kvx_plan_runs(plan, runs, 4, &n) == KVX_OK && n == 2);
  CHECK(runs[0].src0 == 3 && runs[0].dst0 == 10 && runs[0].nblk == 2 && runs[0].tail == BS);
  CHECK(runs[1].src0 == 5 && runs[1].dst0 == 20 && runs[1].nblk == 1 && runs[1].tail == 8);

  /* NHD: each run is one byte range of its region */
  CHECK(kvx_plan_triples(plan, 1, 1, trip, 4, &n) == KVX_OK && n == 2);
  CHECK(trip[0].src_off == 3 * BLOCK_BYTES && trip[0].dst_off == 10 * BLOCK_BYTES && trip[0].len == 2 * BLOCK_BYTES);
  CHECK(trip[1].src_off == 5 * BLOCK_BYTES && trip[1].dst_off == 20 * BLOCK_BYTES && trip[1].len == 8 * TOKEN_BYTES);

  CHECK(kvx_plan_bytes(plan, &rd, &wr) == KVX_OK && rd == 2 * 40 * TOKEN_BYTES && wr == rd);
  CHECK(kvx_staging_bytes(plan, 0, L, &stg) == KVX_OK && stg == (int64_t)L * 2 * 40 * TOKEN_BYTES);
  CHECK(kvx_plan_wait(plan) == KVX_OK); /* nothing uploaded */
  CHECK(kvx_push_layer(plan, 0, NULL, NULL) == KVX_E_INVAL); /* host-only plan: no device calls */

  /* error classes, with the output left untouched */
  CHECK(kvx_plan(src, dst, 1, &tokens, offsets, offsets, src_ids, dup_ids, KVX_PLAN_HOST_ONLY, NULL, &bad) ==
        KVX_E_DUPDST);
  CHECK(bad == NULL && strlen(kvx_last_error()) > 0);
  CHECK(kvx_plan(src, dst, 1, &tokens, offsets, offsets, far_ids, dst_ids, KVX_PLAN_HOST_ONLY, NULL, &bad) ==
        KVX_E_RANGE);
  CHECK(kvx_plan(src, src, 1, &tokens, offsets, offsets, src_ids, dst_ids, KVX_PLAN_HOST_ONLY, NULL, &bad) ==
        KVX_E_INVAL);
  CHECK(bad == NULL);
  CHECK(strcmp(kvx_status_str(KVX_E_RANGE), "KVX_E_RANGE") == 0);

  kvx_plan_destroy(plan);
  kvx_pool_destroy(src);
  kvx_pool_destroy(dst);
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
