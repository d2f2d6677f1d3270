/*
 * Drives the CPU oracle (oracle/c128_oracle.c) through every cache format and its early-exit
 * paths on small deterministic inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py).  It checks the status of each
 * token and that no byte outside the records of written tokens changes.  Test infrastructure.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_compress_store_fmt(
    int64_t head, int indexer, int64_t compress_ratio, int64_t overlap, int64_t state_width,
    const float* state, int64_t n_state_blocks, int64_t state_bs, int64_t s0, int64_t s1,
    const int32_t* block_table, int64_t bt_rows, int64_t bt_cols, int64_t bt_stride,
    const int32_t* token_to_req, const int32_t* positions, const int32_t* slot_mapping,
    int64_t T, const float* rms_w, double eps, const float* cos_sin, int64_t cs_rows,
    int64_t cs_stride, uint8_t* k_cache, int64_t kv_bs, int64_t kv_stride0, int64_t n_kv_blocks,
    const int32_t* kv_slot_mapping, double* out_compressed, double* out_absnorm,
    double* out_normed, int32_t* out_status, int64_t t_lo, int64_t t_hi, int nthreads);

enum { NB = 64, SBS = 8, COLS = 64, T = 8, KVB = 4, KVBS = 4, CSR = 1024 };

static int failures = 0;
#define CHECK(c)                                                           \
  do {                                                                     \
    if (!(c)) {                                                            \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

/* One format: head, cache format code, ratio, overlap, row floats, bytes per cache slot,
   data bytes of a record (the rest of the slot is its scale part). */
static void one(const char* name, int64_t head, int fmt, int64_t cr, int64_t ov, int64_t row,
                int64_t slot_bytes, int64_t rec_bytes) {
  const int64_t s1 = row, s0 = SBS * row;
  float* state = malloc(sizeof(float) * NB * s0);
  for (int64_t i = 0; i < NB * s0; ++i) state[i] = (float)sin(0.37 * (double)i) * 2.0f;
  int32_t bt[T * COLS];
  for (int i = 0; i < T * COLS; ++i) bt[i] = (i * 7 + 3) % NB;
  float* w = malloc(sizeof(float) * head);
  for (int j = 0; j < head; ++j) w[j] = 1.0f + 0.01f * (float)j;
  float* cs = malloc(sizeof(float) * CSR * 64);
  for (int i = 0; i < CSR * 64; ++i) cs[i] = (float)cos(0.01 * (double)i);
  /* tokens: boundary tokens (the first window, and later ones), a non-boundary token, a
     negative state slot, an out-of-range request, an out-of-range block id, a negative kv
     slot, and an out-of-range kv slot */
  int32_t req[T] = {0, 1, 2, 3, 4, 5, 6, 7};
  int32_t pos[T], slot[T] = {0, 0, 0, -1, 0, 0, 0, 0}, kv[T] = {0, 5, 9, 2, 3, 4, -1, 99};
  for (int t = 0; t < T; ++t) pos[t] = (int32_t)(cr * (1 + (t % 3)) - 1);
  pos[2] = (int32_t)(cr * 2 - 2); /* not a boundary */
  req[4] = T + 3;                 /* no such request */
  bt[5 * COLS + (pos[5] / SBS)] = NB + 1; /* a block id out of range in token 5's window */
  const int64_t stride0 = KVBS * slot_bytes + 8;
  const size_t kc_bytes = (size_t)(KVB * stride0);
  uint8_t* kc = malloc(kc_bytes);
  memset(kc, 0xAB, kc_bytes);
  double* comp = malloc(sizeof(double) * T * head);
  double* absn = malloc(sizeof(double) * T * head);
  double* nrm = malloc(sizeof(double) * T * head);
  int32_t status[T];
  int rc = oracle_compress_store_fmt(head, fmt, cr, ov, (1 + ov) * head, state, NB, SBS, s0, s1, bt,
                                     T, COLS, COLS, req, pos, slot, T, w, 1e-6, cs, CSR, 64, kc,
                                     KVBS, stride0, KVB, kv, comp, absn, nrm, status, 0, T, 3);
  CHECK(rc == 0);
  /* expected: 0, 1 written; 2 not a boundary; 3 negative slot; 4, 5 bad index; 6 no kv slot;
     7 kv slot out of range */
  const int32_t want[T] = {1, 1, 0, 0, -1, -1, 2, -1};
  for (int t = 0; t < T; ++t)
    if (status[t] != want[t]) {
      fprintf(stderr, "%s token %d: status %d, expected %d\n", name, t, status[t], want[t]);
      ++failures;
    }
  /* untouched bytes: only the records of tokens 0 and 1 (slots 0 and 5) may change */
  for (size_t b = 0; b < kc_bytes; ++b) {
    const int64_t blk = (int64_t)b / stride0, in = (int64_t)b % stride0;
    int written = 0;
    for (int t = 0; t < 2; ++t) {
      const int64_t s = kv[t], kb = s / KVBS, ko = s % KVBS;
      if (kb != blk) continue;
      if (in >= ko * rec_bytes && in < (ko + 1) * rec_bytes) written = 1;
      const int64_t sc = slot_bytes - rec_bytes;
      if (in >= KVBS * rec_bytes + ko * sc && in < KVBS * rec_bytes + (ko + 1) * sc) written = 1;
    }
    if (!written && kc[b] != 0xAB) {
      fprintf(stderr, "%s: byte %zu outside the written records changed\n", name, b);
      ++failures;
      break;
    }
  }
  free(state); free(w); free(cs); free(kc); free(comp); free(absn); free(nrm);
}

int main(void) {
  one("C128", 512, 0, 128, 0, 1024, 584, 576);
  one("C4", 512, 0, 4, 1, 2048, 584, 576);
  one("indexer FP8", 128, 1, 4, 1, 512, 132, 128);
  one("indexer MXFP4", 128, 2, 4, 1, 512, 68, 64);
  if (failures) return 1;
  printf("oracle driver ok\n");
  return 0;
}
