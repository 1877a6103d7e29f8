/* A C99 consumer of the transfer state machine ABI (kvx_xfer.h), host-only:
 * three scenarios worked by hand from the pages' steps.
 *   1. Prefill first ([PUSH] "Implementierungsdetails" step 3, [MORI] §3.2):
 *      layers saved before the consumer registered are deferred, then issued
 *      in layer order at registration; sealed with two writes and both
 *      finished, the request is DONE.
 *   2. Register first, a failed write ([MORI] §3.1): the request is FAILED
 *      and every registered destination block is to be recomputed.
 *   3. Deferral timeout ([MORI] §3.2, default 60 s): a write still deferred
 *      at 59.9 s keeps the request PENDING; at 60.0 s it is EXPIRED.
 * Prints "ok" and exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvx_xfer.h"

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

enum { L = 2, NB = 64, BS = 16, H = 2, D = 64, E = 2 };
#define REGION_BYTES ((uintptr_t)NB * BS * H * D * E)

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

static int32_t state_of(const kvx_xfer* x, uint64_t req) {
  uint32_t attempt = 0;
  int32_t state = -1;
  CHECK(kvx_xfer_status(x, req, &attempt, &state) == KVX_OK);
  return state;
}

int main(void) {
  kvx_pool* prod = make_pool((uintptr_t)1 << 40);
  kvx_pool* cons = make_pool((uintptr_t)1 << 41);
  kvx_xfer_config cfg;
  kvx_xfer* x = NULL;
  int32_t acc = -1;
  uint64_t reqs[4];
  uint32_t atts[4];
  int32_t states[4], layers[4], blocks[4];
  int64_t n = 0;

  memset(&cfg, 0, sizeof cfg);
  cfg.defer_timeout_s = 60.0;
  cfg.transfer_timeout_s = 30.0;
  cfg.flags = KVX_XFER_HOST_ONLY | KVX_XFER_LOG;
  CHECK(kvx_xfer_create(prod, &cfg, NULL, &x) == KVX_OK);

  { /* 1. prefill first */
    const int32_t src[3] = {3, 4, 5}, dst[3] = {10, 11, 20};
    CHECK(kvx_xfer_prefill(x, 7, 1, kvx_tokens_to_move(41, 0), src, 3, 0.0, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_save_layer(x, 7, 1, 0, NULL, 0.1, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_save_layer(x, 7, 1, 1, NULL, 0.2, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_issued(x, 0, reqs, atts, layers, 4, &n) == KVX_OK && n == 0); /* deferred */
    CHECK(kvx_xfer_register(x, 7, 1, cons, dst, 3, 0.3, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_issued(x, 0, reqs, atts, layers, 4, &n) == KVX_OK && n == 2);
    CHECK(reqs[0] == 7 && layers[0] == 0 && reqs[1] == 7 && layers[1] == 1);
    CHECK(kvx_xfer_seal(x, 7, 1, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_save_layer(x, 7, 1, 1, NULL, 0.4, &acc) == KVX_OK && acc == 0); /* after seal */
    CHECK(kvx_xfer_complete(x, 7, 1, 0, 1) == KVX_OK);
    CHECK(kvx_xfer_poll(x, 0.5) == KVX_OK && state_of(x, 7) == KVX_REQ_PENDING);
    CHECK(kvx_xfer_complete(x, 7, 1, 1, 1) == KVX_OK);
    CHECK(kvx_xfer_poll(x, 0.6) == KVX_OK && state_of(x, 7) == KVX_REQ_DONE);
    CHECK(kvx_xfer_recompute_blocks(x, 7, blocks, 4, &n) == KVX_OK && n == 0);
  }
  { /* 2. register first, a failed write */
    const int32_t src[2] = {40, 41}, dst[2] = {30, 31};
    CHECK(kvx_xfer_register(x, 9, 1, cons, dst, 2, 1.0, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_prefill(x, 9, 1, 20, src, 2, 1.1, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_save_layer(x, 9, 1, 0, NULL, 1.2, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_issued(x, 2, reqs, atts, layers, 4, &n) == KVX_OK && n == 1 && reqs[0] == 9 && layers[0] == 0);
    CHECK(kvx_xfer_complete(x, 9, 1, 0, 0) == KVX_OK);
    CHECK(kvx_xfer_poll(x, 1.3) == KVX_OK && state_of(x, 9) == KVX_REQ_FAILED);
    CHECK(kvx_xfer_recompute_blocks(x, 9, blocks, 4, &n) == KVX_OK && n == 2 && blocks[0] == 30 && blocks[1] == 31);
  }
  { /* 3. deferral timeout */
    const int32_t src[1] = {50};
    CHECK(kvx_xfer_prefill(x, 11, 1, 10, src, 1, 0.0, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_save_layer(x, 11, 1, 0, NULL, 0.0, &acc) == KVX_OK && acc == 1);
    CHECK(kvx_xfer_poll(x, 59.9) == KVX_OK && state_of(x, 11) == KVX_REQ_PENDING);
    CHECK(kvx_xfer_poll(x, 60.0) == KVX_OK && state_of(x, 11) == KVX_REQ_EXPIRED);
  }
  /* finished requests in increasing ID */
  CHECK(kvx_xfer_pop_finished(x, reqs, atts, states, 4, &n) == KVX_OK && n == 3);
  CHECK(reqs[0] == 7 && states[0] == KVX_REQ_DONE && reqs[1] == 9 && states[1] == KVX_REQ_FAILED &&
        reqs[2] == 11 && states[2] == KVX_REQ_EXPIRED);
  CHECK(kvx_xfer_forget(x, 7) == KVX_OK && kvx_xfer_forget(x, 7) == KVX_E_RANGE);

  kvx_xfer_destroy(x);
  kvx_pool_destroy(prod);
  kvx_pool_destroy(cons);
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
