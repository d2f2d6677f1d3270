/*
 * A plain C11 consumer of include/dsv4_c128.h, with no Python and no torch.  It exercises the
 * host-only part of the boundary (validation, workspace sizing, the version and the error
 * message), which needs no GPU: descriptors point into host arrays that validation never reads.
 * Prints "abi consumer ok" and exits 0 when every check holds; otherwise names the first check
 * that failed and exits 1.
 */
#include <stdalign.h>
#include <stdio.h>
#include <string.h>

#include "dsv4_c128.h"

static int failures = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

/* Backing storage for descriptors; validation only looks at the pointer values. */
alignas(256) static unsigned char storage[1 << 16];

static dsv4_tensor tensor(int32_t dtype, int32_t ndim, const int64_t* shape) {
  dsv4_tensor t;
  memset(&t, 0, sizeof t);
  t.data = storage;
  t.dtype = dtype;
  t.ndim = ndim;
  int64_t stride = 1;
  for (int i = ndim - 1; i >= 0; --i) {
    t.shape[i] = shape[i];
    t.stride[i] = stride;
    stride *= shape[i];
  }
  return t;
}

typedef struct args {
  dsv4_tensor state, table, req, pos, slot, w, cs, kc, kvslot;
  float eps;
} args;

/* Valid descriptors for T tokens; `row` is the state row width and `head` the output width. */
static args make(int64_t T, int64_t bs, int64_t row, int64_t head, int64_t rec) {
  args a;
  const int64_t st[3] = {32, bs, row}, bt[2] = {T, 64}, tok[1] = {T}, w[1] = {head},
                cs[2] = {128, 64}, kc[3] = {4, 16, rec};
  a.state = tensor(DSV4_F32, 3, st);
  a.table = tensor(DSV4_I32, 2, bt);
  a.req = tensor(DSV4_I32, 1, tok);
  a.pos = tensor(DSV4_I32, 1, tok);
  a.slot = tensor(DSV4_I32, 1, tok);
  a.w = tensor(DSV4_F32, 1, w);
  a.cs = tensor(DSV4_F32, 2, cs);
  a.kc = tensor(DSV4_U8, 3, kc);
  a.kvslot = tensor(DSV4_I32, 1, tok);
  a.eps = 1e-6f;
  return a;
}

typedef int (*validate_fn)(const dsv4_tensor*, const dsv4_tensor*, const dsv4_tensor*,
                           const dsv4_tensor*, const dsv4_tensor*, const dsv4_tensor*, float,
                           const dsv4_tensor*, const dsv4_tensor*, const dsv4_tensor*);

static int run(validate_fn f, const args* a) {
  return f(&a->state, &a->table, &a->req, &a->pos, &a->slot, &a->w, a->eps, &a->cs, &a->kc,
           &a->kvslot);
}

int main(void) {
  CHECK(dsv4_abi_version() == DSV4_ABI_VERSION);

  /* C128: state [S, 8, 1024], rms_w [512], k_cache rows of 584 bytes. */
  args a = make(4, 8, 1024, 512, 584);
  CHECK(run(dsv4_c128_validate, &a) == DSV4_OK);
  CHECK(strcmp(dsv4_last_error(), "") == 0);

  args b = a;
  b.state.shape[1] = 4; /* C128 state blocks hold 8 rows */
  b.state.stride[0] = 4 * 1024;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_SHAPE);
  CHECK(strlen(dsv4_last_error()) > 0);

  b = a;
  b.pos.dtype = DSV4_F32;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_DTYPE);

  b = a;
  b.kc.ndim = 2;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_RANK);

  b = a;
  b.state.stride[2] = 2;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_STRIDE);

  b = a;
  b.state.data = storage + 4; /* state rows must be 16-byte aligned */
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_ALIGN);

  b = a;
  b.w.data = NULL;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_NULL);

  /* Strides: negative on a dimension longer than 1, or a span beyond 2^48 bytes, whatever the
     products of shape and stride would be in 64 bits. */
  b = a;
  b.state.stride[0] = -8192;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_STRIDE);
  b = a;
  b.state.stride[0] = INT64_MAX;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_STRIDE);
  b = a;
  b.kc.stride[0] = INT64_MAX / 2;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_STRIDE);
  b = a;
  b.table.shape[0] = INT32_MAX;
  b.table.stride[0] = (int64_t)1 << 40;
  b.req.shape[0] = b.pos.shape[0] = b.slot.shape[0] = b.kvslot.shape[0] = DSV4_MAX_TOKENS;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_STRIDE);
  b.table.stride[0] = 64;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_OK);
  b.req.shape[0] = b.pos.shape[0] = b.slot.shape[0] = b.kvslot.shape[0] = DSV4_MAX_TOKENS + 1;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_ERR_SHAPE);
  b = a;
  b.table.shape[0] = 1; /* a row stride of a single row is never used */
  b.table.stride[0] = INT64_MIN;
  CHECK(run(dsv4_c128_validate, &b) == DSV4_OK);

  /* A passing call clears the message. */
  CHECK(run(dsv4_c128_validate, &a) == DSV4_OK);
  CHECK(strcmp(dsv4_last_error(), "") == 0);

  /* C4: state [S, bs, 2048] with any block size. */
  for (int64_t bs = 1; bs <= 16; bs *= 2) {
    args c = make(4, bs, 2048, 512, 584);
    CHECK(run(dsv4_c4_validate, &c) == DSV4_OK);
    CHECK(run(dsv4_c128_validate, &c) == DSV4_ERR_SHAPE);
  }

  /* Indexer: state [S, bs, 512], rms_w [128], k_cache rows of 132 bytes. */
  args d = make(4, 2, 512, 128, 132);
  CHECK(run(dsv4_indexer_validate, &d) == DSV4_OK);
  d.w.shape[0] = 512;
  CHECK(run(dsv4_indexer_validate, &d) == DSV4_ERR_SHAPE);

  /* Workspace sizing. */
  CHECK(dsv4_c128_workspace_bytes(16, 3) == 0);
  CHECK(dsv4_c128_workspace_bytes(16, 1) == 0);
  CHECK(dsv4_c128_workspace_bytes(16, 4) > 0);
  CHECK(dsv4_c128_workspace_bytes(16, 8) > dsv4_c128_workspace_bytes(16, 4));
  CHECK(dsv4_c128_workspace_bytes(16, 0) == dsv4_c128_workspace_bytes(16, 8));
  CHECK(dsv4_c128_workspace_bytes(1000, 0) == 0);
  CHECK(dsv4_c128_workspace_bytes(100, 0) == 16384 + 100 * 2 * 6144); /* counters + partials */
  CHECK(dsv4_c128_workspace_bytes(4097, 2) == 0);                      /* above 4096 tokens */
  CHECK(dsv4_c128_varlen_workspace_bytes(0) == 0);
  CHECK(dsv4_c128_varlen_workspace_bytes(1) == 4112); /* 4 * 1025 rounded up to 16 */
  CHECK(dsv4_c128_varlen_workspace_bytes(100) % 16 == 0);
  CHECK(dsv4_c128_varlen_workspace_bytes(100) >= 4 * (1024 + 100));

  if (failures) return 1;
  printf("abi consumer ok\n");
  return 0;
}
