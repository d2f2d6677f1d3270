/*
 * Drives the seeded input generator (synth/synth_gen.c) for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py): a padded pool filled with 1 and
 * with 5 threads must give identical values, leave every padding element unchanged, and the
 * other fill functions must stay inside their outputs.  Test infrastructure.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int synth_fill_pool(float* pool, int64_t n_blocks, int64_t rows_per_block, int64_t stride0,
                    int64_t stride1, int64_t kv_cols, int64_t score_col0, int64_t score_cols,
                    uint64_t seed, double kv_std, const double* score_mean, const double* score_std,
                    double score_mean0, double score_std0, int nthreads);
int synth_fill_normal(float* out, int64_t n, uint64_t seed, uint64_t stream, double mean,
                      double std);
int synth_fill_bits(uint64_t* out, int64_t n, uint64_t seed, uint64_t stream);
int synth_fill_uniform(double* out, int64_t n, uint64_t seed, uint64_t stream);

int main(void) {
  enum { NB = 37, RB = 3, KV = 24, SC = 24, ROWPAD = 5, BLKPAD = 11 };
  const int64_t s1 = KV + SC + ROWPAD, s0 = RB * s1 + BLKPAD, n = NB * s0;
  const float sentinel = -12345.0f;
  float* a = malloc(sizeof(float) * n);
  float* b = malloc(sizeof(float) * n);
  double mean[NB], sd[NB];
  for (int i = 0; i < NB; ++i) { mean[i] = 0.1 * i; sd[i] = 1.0 + 0.01 * i; }
  for (int64_t i = 0; i < n; ++i) a[i] = b[i] = sentinel;
  int fails = 0;
  if (synth_fill_pool(a, NB, RB, s0, s1, KV, KV, SC, 99, 1.0, mean, sd, 0.0, 1.0, 1) != 0) ++fails;
  if (synth_fill_pool(b, NB, RB, s0, s1, KV, KV, SC, 99, 1.0, mean, sd, 0.0, 1.0, 5) != 0) ++fails;
  if (memcmp(a, b, sizeof(float) * n) != 0) { fprintf(stderr, "thread count changed values\n"); ++fails; }
  for (int64_t i = 0; i < n; ++i) {
    const int64_t in_blk = i % s0, r = in_blk / s1, c = in_blk % s1;
    const int data = r < RB && c < KV + SC;
    if (!data && a[i] != sentinel) { fprintf(stderr, "padding %lld written\n", (long long)i); ++fails; break; }
    if (data && a[i] == sentinel) { fprintf(stderr, "element %lld not written\n", (long long)i); ++fails; break; }
  }
  float* f = malloc(sizeof(float) * 1001);
  uint64_t* u = malloc(sizeof(uint64_t) * 1001);
  double* d = malloc(sizeof(double) * 1001);
  if (synth_fill_normal(f, 1001, 7, 3, 0.0, 2.0) != 0) ++fails;
  if (synth_fill_bits(u, 1001, 7, 4) != 0) ++fails;
  if (synth_fill_uniform(d, 1001, 7, 5) != 0) ++fails;
  for (int i = 0; i < 1001; ++i)
    if (!(d[i] > 0.0 && d[i] <= 1.0) && !(d[i] >= 0.0 && d[i] < 1.0)) { ++fails; break; }
  free(a); free(b); free(f); free(u); free(d);
  if (fails) return 1;
  printf("synth driver ok\n");
  return 0;
}
