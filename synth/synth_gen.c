/*
 * Seeded synthetic inputs for the C128 compress-store path.
 *
 * This file only draws random numbers: it holds none of the compressor's
 * arithmetic.  Both the CPU oracle and the GPU path read the buffers it
 * fills, so they see byte-identical inputs.
 *
 * Generator: counter-based.  Every value is a pure function of
 * (seed, stream, index), so the result does not depend on the thread count
 * or on the order of work.  The mixing function is the SplitMix64 output
 * finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014).  Normals use the Box-Muller transform in fp64,
 * rounded once to fp32.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

static inline uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

/* 64 random bits for (seed, stream, index). */
uint64_t synth_bits(uint64_t seed, uint64_t stream, uint64_t index) {
  return sm64(sm64(sm64(seed) ^ stream) + index);
}

/* Uniform double in (0, 1]: 53 random bits, never exactly zero. */
static inline double unit_open0(uint64_t key, uint64_t index) {
  return (double)((sm64(key + index) >> 11) + 1) * 0x1.0p-53;
}

/* Standard normal for counter `index` under `key` (Box-Muller, cosine branch). */
static inline double normal_at(uint64_t key, uint64_t index) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unit_open0(key, 2 * index);
  double u2 = unit_open0(key, 2 * index + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return sm64(sm64(seed) ^ stream);
}

/* ---- threaded fill of a paged fp32 pool ------------------------------- */

typedef struct {
  float* pool;
  int64_t rows_per_block, stride0, stride1;
  int64_t kv_cols, score_col0, score_cols;
  int64_t blk_lo, blk_hi;
  uint64_t kv_key, score_key;
  double kv_std;
  const double* score_mean; /* per block, or NULL */
  const double* score_std;  /* per block, or NULL */
  double score_mean0, score_std0;
} pool_job;

static void* pool_worker(void* arg) {
  const pool_job* j = (const pool_job*)arg;
  for (int64_t b = j->blk_lo; b < j->blk_hi; ++b) {
    double smean = j->score_mean ? j->score_mean[b] : j->score_mean0;
    double sstd = j->score_std ? j->score_std[b] : j->score_std0;
    for (int64_t r = 0; r < j->rows_per_block; ++r) {
      float* row = j->pool + b * j->stride0 + r * j->stride1;
      uint64_t grow = (uint64_t)(b * j->rows_per_block + r);
      for (int64_t c = 0; c < j->kv_cols; ++c)
        row[c] = (float)(j->kv_std * normal_at(j->kv_key, grow * (uint64_t)j->kv_cols + (uint64_t)c));
      for (int64_t c = 0; c < j->score_cols; ++c)
        row[j->score_col0 + c] =
            (float)(smean + sstd * normal_at(j->score_key, grow * (uint64_t)j->score_cols + (uint64_t)c));
    }
  }
  return NULL;
}

/*
 * Fill blocks [0, n_blocks) of a pool laid out as
 * pool[b * stride0 + r * stride1 + c] (element strides).
 * Columns [0, kv_cols) get kv_std * N(0,1) (stream 1).
 * Columns [score_col0, score_col0 + score_cols) get mean_b + std_b * N(0,1)
 * (stream 2), where mean_b/std_b come from the per-block arrays when given,
 * else from score_mean0/score_std0.  Padding columns are not touched.
 */
int synth_fill_pool(float* pool, int64_t n_blocks, int64_t rows_per_block, int64_t stride0,
                    int64_t stride1, int64_t kv_cols, int64_t score_col0, int64_t score_cols,
                    uint64_t seed, double kv_std, const double* score_mean, const double* score_std,
                    double score_mean0, double score_std0, int nthreads) {
  if (!pool || n_blocks < 0 || nthreads < 1) return -1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int created[256];
  pool_job jobs[256];
  int64_t per = (n_blocks + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    pool_job* j = &jobs[t];
    created[t] = 0;
    j->pool = pool;
    j->rows_per_block = rows_per_block;
    j->stride0 = stride0;
    j->stride1 = stride1;
    j->kv_cols = kv_cols;
    j->score_col0 = score_col0;
    j->score_cols = score_cols;
    j->blk_lo = (int64_t)t * per < n_blocks ? (int64_t)t * per : n_blocks;
    j->blk_hi = j->blk_lo + per < n_blocks ? j->blk_lo + per : n_blocks;
    j->kv_key = stream_key(seed, 1);
    j->score_key = stream_key(seed, 2);
    j->kv_std = kv_std;
    j->score_mean = score_mean;
    j->score_std = score_std;
    j->score_mean0 = score_mean0;
    j->score_std0 = score_std0;
    if (j->blk_lo >= j->blk_hi) continue;
    if (pthread_create(&th[t], NULL, pool_worker, j) == 0)
      created[t] = 1;
    else
      pool_worker(j); /* no thread available: do the share inline */
  }
  for (int t = 0; t < nthreads; ++t)
    if (created[t]) pthread_join(th[t], NULL);
  return 0;
}

/* out[i] = mean + std * N(0,1) for counter i of (seed, stream); single thread. */
int synth_fill_normal(float* out, int64_t n, uint64_t seed, uint64_t stream, double mean, double std) {
  if (!out && n) return -1;
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + std * normal_at(key, (uint64_t)i));
  return 0;
}

/* out[i] = 64 random bits for counter i of (seed, stream). */
int synth_fill_bits(uint64_t* out, int64_t n, uint64_t seed, uint64_t stream) {
  if (!out && n) return -1;
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = sm64(key + (uint64_t)i);
  return 0;
}

/* out[i] = uniform double in (0, 1] for counter i of (seed, stream). */
int synth_fill_uniform(double* out, int64_t n, uint64_t seed, uint64_t stream) {
  if (!out && n) return -1;
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = unit_open0(key, (uint64_t)i);
  return 0;
}
