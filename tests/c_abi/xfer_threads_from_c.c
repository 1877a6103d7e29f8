/* Calls on one kvx_xfer are serialized internally, so threads may share it:
 * eight POSIX threads drive disjoint requests through one host-only instance
 * at once, each request taking prefill or registration first, two layer
 * saves deferred until the other side arrives, two issued at once, then seal
 * and completion ([PUSH] "Implementierungsdetails" steps 1-3; [MORI] §3.2).
 * Every request must end DONE and every write be logged once.  Pool
 * addresses are made up: host-only plans never dereference them.  Prints
 * "ok" and exits 0 when every check holds. */
#include <pthread.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvx_xfer.h"

enum { T = 8, PER = 40, L = 4, NB = 64, BS = 4 };

static kvx_xfer* X;
static kvx_pool* CONS;
static int not_done = 0;

static kvx_pool* fake_pool(uintptr_t base) {
  void* kb[L];
  void* vb[L];
  kvx_pool_desc d;
  kvx_pool* p = NULL;
  int l;
  for (l = 0; l < L; ++l) {
    kb[l] = (void*)(base + (uintptr_t)(2 * l) * 65536u);
    vb[l] = (void*)(base + (uintptr_t)(2 * l + 1) * 65536u);
  }
  memset(&d, 0, sizeof d);
  d.num_layers = L;
  d.num_blocks = NB;
  d.block_size = BS;
  d.num_heads = 1;
  d.head_dim = 16;
  d.elem_bytes = 1;
  d.layout = KVX_NHD;
  d.k_base = kb;
  d.v_base = vb;
  if (kvx_pool_create(&d, &p) != KVX_OK) {
    fprintf(stderr, "pool: %s\n", kvx_last_error());
    exit(1);
  }
  return p;
}

static void* worker(void* arg) {
  const int t = (int)(intptr_t)arg;
  const int32_t src[2] = {1, 2}, dst[2] = {3, 4};
  int32_t acc, st;
  uint32_t att;
  int k, l;
  for (k = 0; k < PER; ++k) {
    const uint64_t rid = (uint64_t)t * 1000u + (uint64_t)k;
    if (k % 2)
      kvx_xfer_register(X, rid, 0, CONS, dst, 2, 0.0, &acc);
    else
      kvx_xfer_prefill(X, rid, 0, 8, src, 2, 0.0, &acc);
    for (l = 0; l < L / 2; ++l) kvx_xfer_save_layer(X, rid, 0, l, NULL, 0.0, &acc); /* deferred */
    if (k % 2)
      kvx_xfer_prefill(X, rid, 0, 8, src, 2, 0.0, &acc);
    else
      kvx_xfer_register(X, rid, 0, CONS, dst, 2, 0.0, &acc);
    for (l = L / 2; l < L; ++l) kvx_xfer_save_layer(X, rid, 0, l, NULL, 0.0, &acc);
    kvx_xfer_seal(X, rid, 0, &acc);
    for (l = 0; l < L; ++l) kvx_xfer_complete(X, rid, 0, l, 1);
    kvx_xfer_poll(X, 1.0);
    if (kvx_xfer_status(X, rid, &att, &st) != KVX_OK || st != KVX_REQ_DONE)
      __atomic_add_fetch(&not_done, 1, __ATOMIC_RELAXED);
  }
  return NULL;
}

int main(void) {
  kvx_xfer_config cfg = {60.0, 30.0, KVX_XFER_HOST_ONLY | KVX_XFER_LOG};
  pthread_t th[T];
  int64_t n = 0;
  uint64_t* reqs;
  uint32_t* atts;
  int32_t* layers;
  kvx_pool* prod;
  int t;
  prod = fake_pool((uintptr_t)1 << 40);
  CONS = fake_pool((uintptr_t)2 << 40);
  if (kvx_xfer_create(prod, &cfg, NULL, &X) != KVX_OK) return 1;
  for (t = 0; t < T; ++t) pthread_create(&th[t], NULL, worker, (void*)(intptr_t)t);
  for (t = 0; t < T; ++t) pthread_join(th[t], NULL);
  reqs = malloc(sizeof(uint64_t) * T * PER * L);
  atts = malloc(sizeof(uint32_t) * T * PER * L);
  layers = malloc(sizeof(int32_t) * T * PER * L);
  if (!reqs || !atts || !layers) return 1;
  if (kvx_xfer_issued(X, 0, reqs, atts, layers, T * PER * L, &n) != KVX_OK) n = -1;
  free(reqs);
  free(atts);
  free(layers);
  kvx_xfer_destroy(X);
  kvx_pool_destroy(prod);
  kvx_pool_destroy(CONS);
  if (not_done != 0 || n != T * PER * L) {
    fprintf(stderr, "%d requests not DONE, %lld writes logged\n", not_done, (long long)n);
    return 1;
  }
  printf("ok\n");
  return 0;
}
