/* Drives the C ABI of libemb's host layer through its argument checks, with
 * no device: every call below must be decided (accepted as a no-op, or
 * rejected with the documented status code and a message) before the layer
 * touches HIP. Built with the host sanitizers by tests/test_host_sanitizers.py
 * (device-side calls are stubs that abort). Prints "abi harness ok: N checks"
 * and exits 0, or reports the first mismatch and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "emb.h"

static int g_checks = 0;

#define EXPECT(call, code)                                                                  \
  do {                                                                                      \
    int rc_ = (call);                                                                       \
    ++g_checks;                                                                             \
    if (rc_ != (code)) {                                                                    \
      fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, rc_, \
              (int)(code), emb_last_error());                                               \
      return 1;                                                                             \
    }                                                                                       \
    if ((code) != EMB_OK && emb_last_error()[0] == '\0') {                                  \
      fprintf(stderr, "line %d: %s failed without a message\n", __LINE__, #call);          \
      return 1;                                                                             \
    }                                                                                       \
  } while (0)

#define CHECK(cond)                                                      \
  do {                                                                   \
    ++g_checks;                                                          \
    if (!(cond)) {                                                       \
      fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #cond);   \
      return 1;                                                          \
    }                                                                    \
  } while (0)

/* 16-byte aligned, non-null "device" addresses: never dereferenced. */
#define FAKE(k) ((void*)(uintptr_t)(0x100000u + 0x1000u * (unsigned)(k)))

static emb_table_desc desc(int64_t rows, int32_t dim, int32_t slices, int32_t dtype, int state, int master) {
  emb_table_desc d;
  memset(&d, 0, sizeof d);
  d.rows = rows;
  d.dim = dim;
  d.col_slices = slices;
  d.dtype = dtype;
  for (int s = 0; s < slices && s < EMB_MAX_SLICES; ++s) {
    d.weights[s] = FAKE(s);
    d.state[s] = state ? (float*)FAKE(64 + s) : NULL;
    d.master[s] = master ? (float*)FAKE(128 + s) : NULL;
  }
  return d;
}

static int create_rejects(void) {
  emb_ctx* c = (emb_ctx*)FAKE(0);
  emb_table_desc d[3];
  EXPECT(emb_create_tables(NULL, 1, &c), EMB_E_INVAL);
  CHECK(c == NULL);
  d[0] = desc(10, 16, 1, EMB_F32, 1, 0);
  EXPECT(emb_create_tables(d, 1, NULL), EMB_E_INVAL);
  EXPECT(emb_create_tables(d, 0, &c), EMB_E_INVAL);
  EXPECT(emb_create_tables(d, 5000, &c), EMB_E_INVAL);
  d[0] = desc(10, 16, 1, 9, 1, 0);
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_DTYPE);
  d[0] = desc(10, 96, 5, EMB_F32, 1, 0);
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);      /* more slices than EMB_MAX_SLICES */
  d[0] = desc(10, 100, 3, EMB_F32, 1, 0);
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);      /* dim % slices */
  d[0] = desc(10, 6, 1, EMB_F32, 1, 0);
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);      /* 24-byte rows */
  d[0] = desc(10, 512, 1, EMB_F32, 1, 0);
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);      /* rows wider than 1024 bytes */
  d[0] = desc(0, 16, 1, EMB_F32, 1, 0);
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);      /* no rows */
  d[0] = desc((int64_t)1 << 31, 16, 1, EMB_F32, 1, 0);
  d[1] = desc((int64_t)1 << 31, 16, 1, EMB_F32, 1, 0);
  EXPECT(emb_create_tables(d, 2, &c), EMB_E_INVAL);      /* sum of rows >= 2^32 - 1 */
  d[0] = desc(10, 16, 1, EMB_F32, 1, 0);
  d[1] = desc(10, 32, 1, EMB_F32, 1, 0);
  EXPECT(emb_create_tables(d, 2, &c), EMB_E_INVAL);      /* dims differ */
  d[1] = desc(10, 16, 1, EMB_F32, 0, 0);
  EXPECT(emb_create_tables(d, 2, &c), EMB_E_INVAL);      /* state on some tables only */
  d[0] = desc(10, 16, 1, EMB_F32, 0, 1);
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);      /* fp32 master on an fp32 table */
  d[0] = desc(10, 16, 2, EMB_F16, 0, 1);
  d[0].master[1] = NULL;
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);      /* master on one slice only */
  d[0] = desc(10, 16, 1, EMB_BF16, 0, 1);
  d[0].master[0] = (float*)((char*)FAKE(128) + 8);
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);      /* misaligned master */
  d[0] = desc(10, 16, 1, EMB_F32, 0, 0);
  d[0].weights[2] = FAKE(9);
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);      /* pointer of an unused slice */
  d[0] = desc(10, 16, 1, EMB_F32, 0, 0);
  d[0].reserved = 3;
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);
  d[0] = desc(10, 16, 1, EMB_F32, 0, 0);
  d[0].weights[0] = NULL;
  EXPECT(emb_create_tables(d, 1, &c), EMB_E_INVAL);
  return 0;
}

static int calls_on(emb_ctx* c, int has_state) {
  const void* idx = FAKE(200);
  const void* off = FAKE(201);
  float* out = (float*)FAKE(202);
  void* ws = FAKE(256);          /* 256-byte aligned */
  uint32_t* uk = (uint32_t*)FAKE(203);
  int32_t* cnt = (int32_t*)FAKE(204);
  int32_t* inv = (int32_t*)FAKE(205);
  int32_t* nu = (int32_t*)FAKE(206);
  const float* dY = (const float*)FAKE(207);
  int64_t ro[4];

  EXPECT(emb_row_offsets(c, ro), EMB_OK);
  CHECK(ro[0] == 0 && ro[1] == 1000 && ro[2] == 1700 && ro[3] == 1750);
  EXPECT(emb_row_offsets(c, NULL), EMB_E_INVAL);
  const size_t wsb = emb_backward_workspace_bytes(c, 5000, 64);
  CHECK(wsb > 5000u * 8u);
  CHECK(emb_backward_workspace_bytes(c, -1, 64) == 0);
  CHECK(emb_backward_workspace_bytes(c, (int64_t)1 << 31, 64) == 0);
  CHECK(emb_backward_workspace_bytes(NULL, 10, 10) == 0);
  CHECK(emb_hash_bytes(c) > 0);
  CHECK(emb_hash_workspace_bytes(c, 1000) >= 1000u * 36u);
  CHECK(emb_hash_workspace_bytes(c, -5) == 0);

  /* forward: decided before any device call */
  EXPECT(emb_forward_pooled(NULL, idx, off, EMB_I32, 10, 4, EMB_POOL_SUM, out, NULL), EMB_E_INVAL);
  EXPECT(emb_forward_pooled(c, idx, off, 7, 10, 4, EMB_POOL_SUM, out, NULL), EMB_E_DTYPE);
  EXPECT(emb_forward_pooled(c, idx, off, EMB_I32, 10, 4, 9, out, NULL), EMB_E_DTYPE);
  EXPECT(emb_forward_pooled(c, idx, off, EMB_I32, -1, 4, EMB_POOL_SUM, out, NULL), EMB_E_INVAL);
  EXPECT(emb_forward_pooled(c, idx, off, EMB_I32, (int64_t)1 << 31, 4, EMB_POOL_SUM, out, NULL), EMB_E_INVAL);
  EXPECT(emb_forward_pooled(c, idx, off, EMB_I32, 10, 0, EMB_POOL_SUM, out, NULL), EMB_E_INVAL);
  EXPECT(emb_forward_pooled(c, idx, off, EMB_I32, 0, 0, EMB_POOL_SUM, out, NULL), EMB_OK);   /* nothing to do */
  EXPECT(emb_forward_pooled(c, idx, NULL, EMB_I32, 10, 4, EMB_POOL_SUM, out, NULL), EMB_E_INVAL);
  EXPECT(emb_forward_pooled(c, NULL, off, EMB_I32, 10, 4, EMB_POOL_SUM, out, NULL), EMB_E_INVAL);
  EXPECT(emb_forward_pooled(c, idx, off, EMB_I32, 10, 4, EMB_POOL_SUM, (float*)((char*)out + 4), NULL),
         EMB_E_INVAL);
  EXPECT(emb_forward_pooled_unique(c, idx, off, EMB_I32, 10, 4, EMB_POOL_SUM, ws, FAKE(208), 1 << 20, out, NULL),
         EMB_E_STATE);       /* no dedup done ahead */

  /* backward / dedup */
  EXPECT(emb_backward_unique_reduce(c, idx, off, EMB_I64, 5000, 64, EMB_POOL_MEAN, dY, ws, wsb - 1, uk, cnt, inv,
                                    nu, NULL, NULL), EMB_E_WORKSPACE);
  EXPECT(emb_backward_unique_reduce(c, idx, off, EMB_I64, 5000, 64, EMB_POOL_MEAN, dY, (char*)ws + 16, wsb, uk,
                                    cnt, inv, nu, NULL, NULL), EMB_E_INVAL);        /* misaligned ws */
  EXPECT(emb_backward_unique_reduce(c, idx, off, EMB_I64, 5000, 64, EMB_POOL_MEAN, NULL, ws, wsb, uk, cnt, inv,
                                    nu, NULL, NULL), EMB_E_INVAL);                  /* no dY */
  EXPECT(emb_backward_unique_reduce(c, idx, off, EMB_I64, 5000, 64, EMB_POOL_MEAN, (const float*)((char*)dY + 4),
                                    ws, wsb, uk, cnt, inv, nu, NULL, NULL), EMB_E_INVAL);
  EXPECT(emb_backward_unique_reduce(c, idx, off, EMB_I64, 5000, 64, EMB_POOL_MEAN, dY, ws, wsb, NULL, cnt, inv,
                                    nu, NULL, NULL), EMB_E_INVAL);
  EXPECT(emb_backward_unique_reduce(c, idx, off, 3, 5000, 64, EMB_POOL_MEAN, dY, ws, wsb, uk, cnt, inv, nu, NULL,
                                    NULL), EMB_E_DTYPE);
  EXPECT(emb_backward_dedup(c, idx, off, EMB_I32, 5000, 64, EMB_POOL_SUM, ws, wsb, uk, cnt, inv, NULL, NULL),
         EMB_E_INVAL);
  EXPECT(emb_backward_dedup(c, idx, off, EMB_I32, 5000, 0, EMB_POOL_SUM, ws, wsb, uk, cnt, inv, nu, NULL),
         EMB_E_INVAL);
  EXPECT(emb_backward_dedup(c, idx, off, EMB_I32, 5000, 1 << 30, EMB_POOL_SUM, ws, wsb, uk, cnt, inv, nu, NULL),
         EMB_E_INVAL);      /* B*T*dim >= 2^32 */

  /* update: nothing to apply yet, and argument checks */
  EXPECT(emb_sparse_update(c, 5, 0.1f, 1e-8f, ws, dY, NULL, NULL), EMB_E_DTYPE);
  EXPECT(emb_sparse_update(c, EMB_OPT_SGD, 0.1f, 0.f, ws, dY, NULL, NULL), EMB_E_STATE);
  EXPECT(emb_sparse_update(c, EMB_OPT_ADAGRAD, 0.1f, 1e-8f, ws, dY, NULL, NULL),
         has_state ? EMB_E_STATE : EMB_E_INVAL);
  EXPECT(emb_backward_atomic_reduce(c, off, EMB_I32, 10, 4, EMB_POOL_SUM, dY, inv, nu, NULL, NULL), EMB_E_INVAL);
  EXPECT(emb_backward_atomic_reduce(c, off, EMB_I32, 0, 4, EMB_POOL_SUM, dY, inv, nu, (float*)out, NULL), EMB_OK);

  /* routing: the map is host state; packing needs a backward first */
  emb_shard_rule r[3] = {{EMB_SHARD_TABLE, 1}, {EMB_SHARD_ROW_CYCLIC, 0}, {EMB_SHARD_ROW_BLOCK, 0}};
  EXPECT(emb_set_shard_map(c, r, 0), EMB_E_INVAL);
  EXPECT(emb_set_shard_map(c, r, EMB_MAX_SHARDS + 1), EMB_E_INVAL);
  EXPECT(emb_set_shard_map(c, r, 1), EMB_E_INVAL);      /* shard 1 of 1 */
  r[2].shard = 1;
  EXPECT(emb_set_shard_map(c, r, 4), EMB_E_INVAL); /* row blocks take shard 0 */
  r[2].shard = 0;
  r[1].kind = 7;
  EXPECT(emb_set_shard_map(c, r, 4), EMB_E_INVAL);
  r[1].kind = EMB_SHARD_ROW_CYCLIC;
  EXPECT(emb_set_shard_map(c, r, 4), EMB_OK);
  EXPECT(emb_pack_by_shard(c, ws, NULL, uk, cnt, inv, NULL, NULL), EMB_E_STATE);

  /* hash-keyed lookup: nothing attached */
  const int64_t* ids = (const int64_t*)FAKE(209);
  EXPECT(emb_hash_attach(c, NULL, 1 << 20, NULL), EMB_E_INVAL);
  EXPECT(emb_hash_attach(c, (char*)FAKE(300) + 16, 1 << 20, NULL), EMB_E_INVAL);   /* not 256-byte aligned */
  EXPECT(emb_hash_attach(c, FAKE(300), 16, NULL), EMB_E_WORKSPACE);
  EXPECT(emb_hash_translate(c, ids, off, EMB_I32, 10, 4, 1, ws, 1 << 20, (void*)inv, NULL), EMB_E_STATE);
  EXPECT(emb_hash_translate_noalloc(c, ids, off, EMB_I32, 10, 4, 1, (void*)inv, NULL), EMB_E_STATE);
  EXPECT(emb_forward_pooled_hashed(c, ids, off, EMB_I32, 10, 4, EMB_POOL_MEAN, out, NULL), EMB_E_STATE);
  EXPECT(emb_hash_rows_used(c, cnt, NULL), EMB_E_STATE);
  EXPECT(emb_hash_rows_used(c, NULL, NULL), EMB_E_INVAL);

  /* misc: the device block does not exist yet, so nothing to check or wait for */
  EXPECT(emb_check_device_error(c, NULL), EMB_OK);
  EXPECT(emb_set_kernel_timing(c, 1), EMB_OK);
  double ms[EMB_K_COUNT];
  int64_t n[EMB_K_COUNT];
  EXPECT(emb_kernel_times(c, ms, n), EMB_OK);
  CHECK(n[EMB_K_FORWARD] == 0 && ms[EMB_K_REDUCE] == 0.0);
  EXPECT(emb_kernel_times(c, NULL, n), EMB_E_INVAL);
  EXPECT(emb_set_kernel_timing(NULL, 1), EMB_E_INVAL);
  EXPECT(emb_init_uniform(NULL, 1, NULL), EMB_E_INVAL);
  return 0;
}

int main(void) {
  if (create_rejects()) return 1;
  emb_table_desc d[3] = {desc(1000, 32, 2, EMB_F16, 1, 1), desc(700, 32, 2, EMB_F16, 1, 1),
                         desc(50, 32, 2, EMB_F16, 1, 1)};
  emb_ctx* c = NULL;
  EXPECT(emb_create_tables(d, 3, &c), EMB_OK);
  CHECK(c != NULL && emb_last_error()[0] == '\0');
  if (calls_on(c, 1)) return 1;
  emb_destroy_tables(c);
  emb_table_desc e[3] = {desc(1000, 16, 1, EMB_F32, 0, 0), desc(700, 16, 1, EMB_F32, 0, 0),
                         desc(50, 16, 1, EMB_F32, 0, 0)};
  EXPECT(emb_create_tables(e, 3, &c), EMB_OK);
  if (calls_on(c, 0)) return 1;
  emb_destroy_tables(c);
  emb_destroy_tables(NULL);
  printf("abi harness ok: %d checks\n", g_checks);
  return 0;
}
