/*
 * CPU ORACLE for the DeepSeek-V4 compress-store paths: the sparse-attention compressors (C128,
 * and C4 with its overlapping window) and the indexer's FP8 compressor.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's
 * cpu_baseline leg use it.  It shares no code with the HIP library.
 *
 * It is a plain, slow, obviously correct statement of what the path
 * computes, in fp64, token by token, following the vLLM API page
 * "fused_compress_quant_cache" (DeepSeek-V4 common ops), kernel
 * `_fused_kv_compress_norm_rope_insert_sparse_attn` and its two-stage twins
 * `_compress_gather_split_sparse_attn` / `_finalize_norm_rope_quant_store_sparse_attn`:
 *
 *   gate    a token is active iff its state slot is >= 0 and (pos+1) % CR == 0
 *           (compress ratio CR = 128, or 4 for the C4 compressor)
 *   gather  window rows q = pos - (1+OV)*CR + 1 .. pos (overlap OV = 0 for C128, 1 for C4),
 *           row q at state[bt[req][q / bs]][q % bs]; rows with q < 0 take no part;
 *           window row i reads its kv at column offset h_i = (i >= CR ? 512 : 0) of the state
 *           row and its score at state_width + h_i (state_width = 512 for C128, 1024 for C4)
 *   pool    c_j = sum_i softmax_i(score_ij) * kv_ij          (per column j < 512)
 *   norm    n_j = c_j / sqrt(mean_j c_j^2 + eps) * w_j
 *   quant   dims < 448: bf16 round trip, per-64 absmax (floor 1e-4), UE8M0
 *           exponent e = ceil(log2(absmax / 448)), e4m3fn codes of x * 2^-e
 *   rope    dims 448..511: interleaved pairs rotated by the table row
 *           (pos // CR) * CR, stored as bf16
 *   insert  kv slot s >= 0: block s / kv_bs, offset s % kv_bs;
 *           576 data bytes at blk*stride0 + off*576,
 *           8 scale bytes (7 exponents + a zero pad) at blk*stride0 + kv_bs*576 + off*8
 *
 * The indexer's compressor (same page, kernel `_fused_kv_compress_norm_rope_insert_indexer_attn`)
 * pools a head of 128 the same way, then, after RMSNorm:
 *   rope    dims 64..127: interleaved pairs rotated by table row (pos // CR) * CR, kept in fp32
 *   quant   all 128 dims, after the rotation: bf16 round trip, one absmax (floor 1e-4),
 *           e = ceil(log2(absmax / 448)), e4m3fn codes of x * 2^-e, and the scale 2^e as fp32
 *   insert  128 code bytes at blk*stride0 + off*128, the fp32 scale at blk*stride0 +
 *           kv_bs*128 + off*4
 *
 * Its MXFP4 variant (same page, kernel `_fused_kv_compress_norm_rope_insert_indexer_mxfp4_attn`)
 * pools, normalises and rotates the same way, then:
 *   round   every rotated value (held in fp32) goes through bf16
 *   quant   four blocks of 32 consecutive dims: absmax (floor 6 * 2^-126), exponent
 *           e = ceil(log2(absmax / 6)) clamped to [-127, 127], E2M1 codes of x * 2^-e
 *   insert  64 bytes at blk*stride0 + off*64, byte p holding dim 2p in its low nibble and
 *           dim 2p+1 in its high nibble; the 4 exponent bytes e + 127 at blk*stride0 +
 *           kv_bs*64 + off*4
 *
 * Readings where the pages leave a point open (each one is listed with its
 * reason in the design notes of the repository):
 *   - int32 index arrays; fp32 rms weight and cos/sin table;
 *   - `.to(bfloat16)` and `.to(float8e4nv)` round to nearest, ties to even;
 *     float8e4nv is the OCP E4M3FN format (bias 7, max 448, no infinities);
 *   - the exponent is the exact ceil(log2) of the fp32 product absmax * fl32(1/448)
 *     (MXFP4: absmax * fl32(1/6));
 *   - the page does not print its E2M1 conversion: E2M1 rounds to nearest, ties to the
 *     even code, keeps the sign (zero included) and saturates at 6, like the E4M3 reading;
 *   - the normalised value is held in fp32 before the bf16 round trip (its
 *     storage type on the page); RoPE rotates the fp64 normalised value and
 *     rounds once to bf16;
 *   - a negative position is inactive;
 *   - an active token with a negative kv slot writes nothing.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HEAD 512        /* head size */
#define NOPE 448        /* FP8 dims */
#define ROPE 64         /* bf16 RoPE dims */
#define HALF_ROPE 32
#define MAX_ROWS 256    /* (1 + overlap) * compress ratio, at most 2 * 128 */
#define QBLOCK 64       /* quantisation block */
#define NQ (NOPE / QBLOCK)
#define RECORD 576      /* 448 fp8 bytes + 64 bf16 */
#define SCALE_DIM 8     /* 7 UE8M0 bytes + 1 pad */
#define FP8_MAX 448.0
#define IDX_HEAD 128    /* indexer head size */
#define IDX_NOPE 64     /* indexer dims before the RoPE dims */
#define IDX_RECORD 128  /* indexer fp8 bytes per token */
#define IDX_SCALE 4     /* one fp32 scale per token */
#define FP4_BLOCK 32    /* MXFP4 quantisation block */
#define FP4_RECORD 64   /* packed E2M1 bytes per token, two dims a byte */
#define FP4_SCALES 4    /* one UE8M0 byte per block */
#define FP4_MAX 6.0

enum { FMT_SPARSE = 0, FMT_INDEXER_FP8 = 1, FMT_INDEXER_MXFP4 = 2 };

/* ------------------------------------------------------------------------
 * Number formats, from their definitions.
 * --------------------------------------------------------------------- */

/*
 * bfloat16 is binary32 with its significand cut to 8 bits (1 implicit + 7
 * stored) and the same exponent range.  Round x (any finite double) to the
 * nearest such value, ties to an even last bit: scale by the spacing of
 * bf16 numbers at x's binade, rint (round-half-even), scale back.  Returns
 * the 16-bit pattern.  Finite inputs below 2^128 only.
 */
uint16_t oracle_bf16_bits(double x) {
  double a = fabs(x);
  double r;
  if (a == 0.0) {
    r = 0.0;
  } else {
    int k;
    frexp(a, &k);             /* a = f * 2^k, f in [0.5, 1) -> binade 2^(k-1) */
    int q = k - 1 - 7;        /* spacing of 8-bit significands in that binade */
    if (q < -133) q = -133;   /* subnormal spacing of binary32 (and of bf16) */
    r = ldexp(rint(ldexp(a, -q)), q);
  }
  float f = (float)r;         /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t h = (uint16_t)(u >> 16);
  if (signbit(x)) h |= 0x8000u;
  return h;
}

double oracle_bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/*
 * OCP 8-bit floating point, E4M3FN: sign, 4 exponent bits (bias 7), 3
 * mantissa bits; subnormals m * 2^-9; largest finite 0x7E = 1.75 * 2^8 = 448.
 * Round |x| <= 448 to nearest, ties to the even code.
 */
uint8_t oracle_e4m3_code(double x) {
  double a = fabs(x);
  uint8_t sign = signbit(x) ? 0x80u : 0x00u;
  unsigned code;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: value = m * 2^-9, m = 0..7; m = 8 is the smallest normal */
    code = (unsigned)rint(ldexp(a, 9));
  } else {
    int k;
    frexp(a, &k);
    int E = k - 1;                                          /* a in [2^E, 2^(E+1)) */
    double m = rint((ldexp(a, -E) - 1.0) * 8.0);            /* 3-bit mantissa, RNE */
    if (m == 8.0) { m = 0.0; E += 1; }
    code = ((unsigned)(E + 7) << 3) | (unsigned)m;
  }
  return (uint8_t)(sign | code);
}

double oracle_e4m3_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/*
 * OCP 4-bit floating point, E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit.  Exponent
 * field 0 holds the subnormals m * 0.5; field E > 0 holds (1 + m/2) * 2^(E-1).  So the eight
 * magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Round |x| (finite) to nearest, ties to the even
 * code; magnitudes beyond 6 saturate to 6.  The sign bit 0x8 follows the sign of x.
 */
uint8_t oracle_e2m1_code(double x) {
  double a = fabs(x);
  unsigned sign = signbit(x) ? 0x8u : 0x0u;
  unsigned code;
  if (a < 1.0) {
    /* subnormal step 0.5; rint = 2 is the smallest normal, 1.0 */
    code = (unsigned)rint(a * 2.0);
  } else {
    int k;
    frexp(a, &k);
    int E = k - 1;                                          /* a in [2^E, 2^(E+1)) */
    double m = rint((ldexp(a, -E) - 1.0) * 2.0);            /* 1-bit mantissa, RNE */
    if (m == 2.0) { m = 0.0; E += 1; }
    code = E > 2 ? 7u : (((unsigned)(E + 1) << 1) | (unsigned)m);
  }
  return (uint8_t)(sign | code);
}

double oracle_e2m1_value(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + m / 2.0, e - 1);
  return s ? -v : v;
}

/* Exact ceil(log2(r)) for a positive finite r. */
int oracle_ceil_log2(double r) {
  int k;
  double f = frexp(r, &k); /* r = f * 2^k, f in [0.5, 1) */
  return (f == 0.5) ? k - 1 : k;
}

/*
 * UE8M0 exponent of one quantisation block from its absmax (of bf16 values):
 * absmax is floored at fl32(1e-4), multiplied by fl32(1/448) in fp32, and
 * e = ceil(log2(that product)).  The product of two fp32 values is exact in
 * fp64, so one cast to float is the fp32 multiply.
 */
int oracle_ue8m0_exponent(double absmax) {
  double floor_ = (double)(float)1e-4;
  double A = absmax > floor_ ? absmax : floor_;
  double inv = (double)(float)(1.0 / FP8_MAX);
  double raw = (double)(float)(A * inv);
  return oracle_ceil_log2(raw);
}

/*
 * UE8M0 exponent of one MXFP4 block from its absmax (of bf16 values): absmax is floored at
 * 6 * 2^-126, multiplied by fl32(1/6) in fp32, e = ceil(log2(that product)), and e is clamped
 * to [-127, 127].  As above, the fp64 product of the two fp32 values is exact, so one cast
 * to float is the fp32 multiply.
 */
int oracle_mxfp4_exponent(double absmax) {
  double floor_ = ldexp(FP4_MAX, -126);
  double A = absmax > floor_ ? absmax : floor_;
  double inv = (double)(float)(1.0 / FP4_MAX);
  double raw = (double)(float)(A * inv);
  int e = oracle_ceil_log2(raw);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

/* ------------------------------------------------------------------------
 * One token.
 * --------------------------------------------------------------------- */

typedef struct {
  int64_t head;                                /* 512 (sparse attention) or 128 (indexer) */
  int indexer;                                 /* FMT_*: the cache format */
  int64_t cr, overlap, state_width;            /* compress ratio, 0/1, score column offset */
  const float* state;
  int64_t n_state_blocks, state_bs, s0, s1;    /* element strides */
  const int32_t* block_table;
  int64_t bt_rows, bt_cols, bt_stride;
  const int32_t* token_to_req;
  const int32_t* positions;
  const int32_t* slot_mapping;
  int64_t T;
  const float* rms_w;
  double eps;
  const float* cos_sin;
  int64_t cs_rows, cs_stride;
  uint8_t* k_cache;
  int64_t kv_bs, kv_stride0, n_kv_blocks;      /* stride in bytes */
  const int32_t* kv_slot_mapping;
  double* out_compressed;  /* [T, 512] or NULL */
  double* out_absnorm;     /* [T, 512] sum_i p_ij |kv_ij|, or NULL */
  double* out_normed;      /* [T, 512] fp64 normalised value, or NULL */
  int32_t* out_status;     /* [T]: 0 inactive, 1 written, 2 active/no write, <0 bad index */
} oracle_args;

enum { ST_INACTIVE = 0, ST_WRITTEN = 1, ST_NO_SLOT = 2, ST_BAD_INDEX = -1 };

/*
 * Indexer record of token t from its normalised values n[0..128): RoPE first (dims 64..127,
 * GPT-J pairs, table row (pos // CR) * CR; the rotated fp64 value is held in fp32, the page's
 * type), then one quantisation block over all 128 dims, then the insert.  On return n holds
 * the values that were quantised (before their bf16 round trip), in fp64.
 */
static int oracle_indexer_insert(const oracle_args* a, int64_t t, int64_t pos, double* n) {
  int64_t kv_slot = a->kv_slot_mapping[t];
  if (kv_slot < 0) return ST_NO_SLOT;
  int64_t kblk = kv_slot / a->kv_bs, koff = kv_slot % a->kv_bs;
  if (kblk >= a->n_kv_blocks) return ST_BAD_INDEX;
  int64_t P = (pos / a->cr) * a->cr;
  if (P >= a->cs_rows) return ST_BAD_INDEX;

  /* RoPE in fp64 on the normalised pairs (64+2m, 65+2m), m < 32 */
  const float* cs = a->cos_sin + P * a->cs_stride;
  double r[IDX_HEAD];
  for (int j = 0; j < IDX_NOPE; ++j) r[j] = n[j];
  for (int m = 0; m < HALF_ROPE; ++m) {
    double x = n[IDX_NOPE + 2 * m], y = n[IDX_NOPE + 2 * m + 1];
    double C = cs[m], S = cs[HALF_ROPE + m];
    r[IDX_NOPE + 2 * m] = x * C - y * S;
    r[IDX_NOPE + 2 * m + 1] = y * C + x * S;
  }

  /* one quantisation block: fp32, bf16 round trip, absmax, UE8M0 exponent, codes, fp32 scale */
  uint8_t* blockp = a->k_cache + kblk * a->kv_stride0;
  uint8_t* data = blockp + koff * IDX_RECORD;
  uint8_t* scale = blockp + a->kv_bs * IDX_RECORD + koff * IDX_SCALE;
  double u[IDX_HEAD], amax = 0.0;
  for (int j = 0; j < IDX_HEAD; ++j) {
    u[j] = oracle_bf16_value(oracle_bf16_bits((double)(float)r[j]));
    if (fabs(u[j]) > amax) amax = fabs(u[j]);
  }
  int e = oracle_ue8m0_exponent(amax);
  for (int j = 0; j < IDX_HEAD; ++j) {
    double x = ldexp(u[j], -e);
    if (x > FP8_MAX) x = FP8_MAX;
    if (x < -FP8_MAX) x = -FP8_MAX;
    data[j] = oracle_e4m3_code(x);
  }
  float sv = (float)ldexp(1.0, e); /* exact: -22 <= e <= 120 */
  memcpy(scale, &sv, 4);            /* little-endian host, as the device */
  for (int j = 0; j < IDX_HEAD; ++j) n[j] = r[j];
  return ST_WRITTEN;
}

/*
 * MXFP4 indexer record of token t from its normalised values n[0..128): the same RoPE as the
 * FP8 record, every rotated value (held in fp32) through bf16, then four blocks of 32
 * consecutive dims, each with its own UE8M0 exponent, two E2M1 codes a byte (even dim in the
 * low nibble).  On return n holds the rotated values (before their bf16 round trip), in fp64.
 */
static int oracle_indexer_mxfp4_insert(const oracle_args* a, int64_t t, int64_t pos, double* n) {
  int64_t kv_slot = a->kv_slot_mapping[t];
  if (kv_slot < 0) return ST_NO_SLOT;
  int64_t kblk = kv_slot / a->kv_bs, koff = kv_slot % a->kv_bs;
  if (kblk >= a->n_kv_blocks) return ST_BAD_INDEX;
  int64_t P = (pos / a->cr) * a->cr;
  if (P >= a->cs_rows) return ST_BAD_INDEX;

  /* RoPE in fp64 on the normalised pairs (64+2m, 65+2m), m < 32; dims 0..63 unchanged */
  const float* cs = a->cos_sin + P * a->cs_stride;
  double r[IDX_HEAD];
  for (int j = 0; j < IDX_NOPE; ++j) r[j] = n[j];
  for (int m = 0; m < HALF_ROPE; ++m) {
    double x = n[IDX_NOPE + 2 * m], y = n[IDX_NOPE + 2 * m + 1];
    double C = cs[m], S = cs[HALF_ROPE + m];
    r[IDX_NOPE + 2 * m] = x * C - y * S;
    r[IDX_NOPE + 2 * m + 1] = y * C + x * S;
  }

  uint8_t* blockp = a->k_cache + kblk * a->kv_stride0;
  uint8_t* data = blockp + koff * FP4_RECORD;
  uint8_t* scales = blockp + a->kv_bs * FP4_RECORD + koff * FP4_SCALES;
  double u[IDX_HEAD];
  for (int j = 0; j < IDX_HEAD; ++j) u[j] = oracle_bf16_value(oracle_bf16_bits((double)(float)r[j]));
  for (int g = 0; g < IDX_HEAD / FP4_BLOCK; ++g) {
    double amax = 0.0;
    for (int j = g * FP4_BLOCK; j < (g + 1) * FP4_BLOCK; ++j)
      if (fabs(u[j]) > amax) amax = fabs(u[j]);
    int e = oracle_mxfp4_exponent(amax);
    for (int j = g * FP4_BLOCK; j < (g + 1) * FP4_BLOCK; j += 2) {
      uint8_t lo = oracle_e2m1_code(ldexp(u[j], -e));
      uint8_t hi = oracle_e2m1_code(ldexp(u[j + 1], -e));
      data[j / 2] = (uint8_t)(lo | (hi << 4));
    }
    scales[g] = (uint8_t)(e + 127);
  }
  for (int j = 0; j < IDX_HEAD; ++j) n[j] = r[j];
  return ST_WRITTEN;
}

static int oracle_token(const oracle_args* a, int64_t t, double* c, double* absn, double* n) {
  const int64_t CR = a->cr;
  /* gate */
  int32_t slot = a->slot_mapping[t];
  int64_t pos = a->positions[t];
  if (slot < 0 || pos < 0 || (pos + 1) % CR != 0) return ST_INACTIVE;

  int64_t req = a->token_to_req[t];
  if (req < 0 || req >= a->bt_rows) return ST_BAD_INDEX;
  int64_t nrows = (1 + a->overlap) * CR;
  int64_t start = pos - nrows + 1;
  if ((pos / a->state_bs) >= a->bt_cols) return ST_BAD_INDEX;

  /* gather: row pointers of the window, in window order, already offset to the kv half the
     row contributes (the score of the same row is state_width further on); rows before
     position 0 are left out */
  const float* row[MAX_ROWS];
  int valid[MAX_ROWS];
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t q = start + i;
    valid[i] = q >= 0;
    if (!valid[i]) continue;
    int64_t blk = a->block_table[req * a->bt_stride + q / a->state_bs];
    if (blk < 0 || blk >= a->n_state_blocks) return ST_BAD_INDEX;
    int64_t head_offset = (i >= CR) ? a->head : 0;
    row[i] = a->state + blk * a->s0 + (q % a->state_bs) * a->s1 + head_offset;
  }

  /* pool: softmax over the window rows of each score column, weights applied to kv */
  const int64_t SW = a->state_width;
  const int64_t H = a->head;
  for (int j = 0; j < H; ++j) {
    double M = -INFINITY;
    for (int64_t i = 0; i < nrows; ++i) {
      if (!valid[i]) continue;
      double s = row[i][SW + j];
      if (s > M) M = s;
    }
    double w[MAX_ROWS], L = 0.0;
    for (int64_t i = 0; i < nrows; ++i) {
      w[i] = valid[i] ? exp((double)row[i][SW + j] - M) : 0.0;
      L += w[i];
    }
    double num = 0.0, an = 0.0;
    for (int64_t i = 0; i < nrows; ++i) {
      if (!valid[i]) continue;
      double p = w[i] / L;
      num += p * (double)row[i][j];
      an += p * fabs((double)row[i][j]);
    }
    c[j] = num;
    absn[j] = an;
  }

  /* RMSNorm */
  double ss = 0.0;
  for (int j = 0; j < H; ++j) ss += c[j] * c[j];
  double rrms = 1.0 / sqrt(ss / H + a->eps);
  for (int j = 0; j < H; ++j) n[j] = c[j] * rrms * (double)a->rms_w[j];
  if (a->indexer == FMT_INDEXER_MXFP4) return oracle_indexer_mxfp4_insert(a, t, pos, n);
  if (a->indexer == FMT_INDEXER_FP8) return oracle_indexer_insert(a, t, pos, n);

  int64_t kv_slot = a->kv_slot_mapping[t];
  if (kv_slot < 0) return ST_NO_SLOT;
  int64_t kblk = kv_slot / a->kv_bs, koff = kv_slot % a->kv_bs;
  if (kblk >= a->n_kv_blocks) return ST_BAD_INDEX;
  int64_t P = (pos / CR) * CR;
  if (P >= a->cs_rows) return ST_BAD_INDEX;

  uint8_t* blockp = a->k_cache + kblk * a->kv_stride0;
  uint8_t* data = blockp + koff * RECORD;
  uint8_t* scales = blockp + a->kv_bs * RECORD + koff * SCALE_DIM;

  /* quant of the nope dims: bf16 round trip of the fp32 normalised value */
  double u[NOPE];
  for (int j = 0; j < NOPE; ++j) u[j] = oracle_bf16_value(oracle_bf16_bits((double)(float)n[j]));
  for (int g = 0; g < NQ; ++g) {
    double amax = 0.0;
    for (int j = g * QBLOCK; j < (g + 1) * QBLOCK; ++j)
      if (fabs(u[j]) > amax) amax = fabs(u[j]);
    int e = oracle_ue8m0_exponent(amax);
    for (int j = g * QBLOCK; j < (g + 1) * QBLOCK; ++j) {
      double x = ldexp(u[j], -e);
      if (x > FP8_MAX) x = FP8_MAX;
      if (x < -FP8_MAX) x = -FP8_MAX;
      data[j] = oracle_e4m3_code(x);
    }
    int byte = e + 127;
    scales[g] = (uint8_t)(byte < 0 ? 0 : (byte > 255 ? 255 : byte));
  }
  scales[NQ] = 0;

  /* RoPE: GPT-J interleaved pairs (448+2m, 449+2m), angle row of the window's first position */
  const float* cs = a->cos_sin + P * a->cs_stride;
  for (int m = 0; m < HALF_ROPE; ++m) {
    double x = n[NOPE + 2 * m], y = n[NOPE + 2 * m + 1];
    double C = cs[m], S = cs[HALF_ROPE + m];
    uint16_t hx = oracle_bf16_bits(x * C - y * S);
    uint16_t hy = oracle_bf16_bits(y * C + x * S);
    uint8_t* o = data + NOPE + 4 * m; /* little-endian bf16 pairs */
    o[0] = (uint8_t)(hx & 0xFF);
    o[1] = (uint8_t)(hx >> 8);
    o[2] = (uint8_t)(hy & 0xFF);
    o[3] = (uint8_t)(hy >> 8);
  }
  return ST_WRITTEN;
}

typedef struct {
  const oracle_args* a;
  int64_t lo, hi;
} oracle_job;

static void* oracle_worker(void* p) {
  const oracle_job* jb = (const oracle_job*)p;
  const oracle_args* a = jb->a;
  double c[HEAD], absn[HEAD], n[HEAD];
  const int64_t H = a->head;
  const size_t row = (size_t)H * sizeof(double);
  for (int64_t t = jb->lo; t < jb->hi; ++t) {
    for (int j = 0; j < HEAD; ++j) c[j] = absn[j] = n[j] = NAN;
    int st = oracle_token(a, t, c, absn, n);
    if (a->out_status) a->out_status[t] = st;
    if (st == ST_WRITTEN || st == ST_NO_SLOT) {
      if (a->out_compressed) memcpy(a->out_compressed + t * H, c, row);
      if (a->out_absnorm) memcpy(a->out_absnorm + t * H, absn, row);
      if (a->out_normed) memcpy(a->out_normed + t * H, n, row);
    }
  }
  return NULL;
}

/*
 * Run the oracle over tokens [t_lo, t_hi) with `nthreads` threads, for compress ratio
 * `compress_ratio`, overlap 0 or 1 and the score column offset `state_width` (>= the kv
 * columns (1 + overlap) * 512 a row holds).  Tokens
 * are independent; each thread takes a contiguous range.  The k_cache is
 * modified in place exactly where the path writes.  Diagnostics arrays (may
 * be NULL) are [T, 512] fp64, rows of tokens that do not pass the gate are
 * left untouched.  Returns 0, or -1 on bad arguments.
 */
int oracle_compress_store_fmt(
    int64_t head, int indexer, int64_t compress_ratio, int64_t overlap, int64_t state_width,
    const float* state, int64_t n_state_blocks, int64_t state_bs, int64_t s0, int64_t s1,
    const int32_t* block_table, int64_t bt_rows, int64_t bt_cols, int64_t bt_stride,
    const int32_t* token_to_req, const int32_t* positions, const int32_t* slot_mapping,
    int64_t T, const float* rms_w, double eps, const float* cos_sin, int64_t cs_rows,
    int64_t cs_stride, uint8_t* k_cache, int64_t kv_bs, int64_t kv_stride0, int64_t n_kv_blocks,
    const int32_t* kv_slot_mapping, double* out_compressed, double* out_absnorm,
    double* out_normed, int32_t* out_status, int64_t t_lo, int64_t t_hi, int nthreads) {
  if (!state || !block_table || !token_to_req || !positions || !slot_mapping || !rms_w ||
      !cos_sin || !k_cache || !kv_slot_mapping || state_bs < 1 || kv_bs < 1 || T < 0 ||
      t_lo < 0 || t_hi > T || t_lo > t_hi || nthreads < 1 || compress_ratio < 1 ||
      (overlap != 0 && overlap != 1) || (1 + overlap) * compress_ratio > MAX_ROWS ||
      indexer < FMT_SPARSE || indexer > FMT_INDEXER_MXFP4 ||
      (indexer ? head != IDX_HEAD : head != HEAD) || state_width < (1 + overlap) * head)
    return -1;
  oracle_args a = {head, indexer, compress_ratio, overlap, state_width, state, n_state_blocks, state_bs, s0, s1, block_table, bt_rows, bt_cols,
                   bt_stride, token_to_req, positions, slot_mapping, T, rms_w, eps, cos_sin,
                   cs_rows, cs_stride, k_cache, kv_bs, kv_stride0, n_kv_blocks, kv_slot_mapping,
                   out_compressed, out_absnorm, out_normed, out_status};
  if (nthreads > 256) nthreads = 256;
  int64_t n = t_hi - t_lo;
  if (nthreads > n) nthreads = n > 0 ? (int)n : 1;
  pthread_t th[256];
  int created[256];
  oracle_job jobs[256];
  int64_t per = (n + nthreads - 1) / nthreads;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].a = &a;
    jobs[i].lo = t_lo + (int64_t)i * per < t_hi ? t_lo + (int64_t)i * per : t_hi;
    jobs[i].hi = jobs[i].lo + per < t_hi ? jobs[i].lo + per : t_hi;
    created[i] = 0;
    if (jobs[i].lo >= jobs[i].hi) continue;
    if (nthreads > 1 && pthread_create(&th[i], NULL, oracle_worker, &jobs[i]) == 0)
      created[i] = 1;
    else
      oracle_worker(&jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i)
    if (created[i]) pthread_join(th[i], NULL);
  return 0;
}


/* The sparse-attention compressors (head 512): compress ratio, overlap 0 or 1, state width. */
int oracle_compress_store(
    int64_t compress_ratio, int64_t overlap, int64_t state_width, const float* state,
    int64_t n_state_blocks, int64_t state_bs, int64_t s0, int64_t s1,
    const int32_t* block_table, int64_t bt_rows, int64_t bt_cols, int64_t bt_stride,
    const int32_t* token_to_req, const int32_t* positions, const int32_t* slot_mapping,
    int64_t T, const float* rms_w, double eps, const float* cos_sin, int64_t cs_rows,
    int64_t cs_stride, uint8_t* k_cache, int64_t kv_bs, int64_t kv_stride0, int64_t n_kv_blocks,
    const int32_t* kv_slot_mapping, double* out_compressed, double* out_absnorm,
    double* out_normed, int32_t* out_status, int64_t t_lo, int64_t t_hi, int nthreads) {
  return oracle_compress_store_fmt(HEAD, 0, compress_ratio, overlap, state_width, state,
                                   n_state_blocks, state_bs, s0, s1, block_table, bt_rows, bt_cols,
                                   bt_stride, token_to_req, positions, slot_mapping, T, rms_w, eps,
                                   cos_sin, cs_rows, cs_stride, k_cache, kv_bs, kv_stride0,
                                   n_kv_blocks, kv_slot_mapping, out_compressed, out_absnorm,
                                   out_normed, out_status, t_lo, t_hi, nthreads);
}

/* The C128 path: compress ratio 128, no overlap, state width 512. */
int oracle_c128_compress_store(
    const float* state, int64_t n_state_blocks, int64_t state_bs, int64_t s0, int64_t s1,
    const int32_t* block_table, int64_t bt_rows, int64_t bt_cols, int64_t bt_stride,
    const int32_t* token_to_req, const int32_t* positions, const int32_t* slot_mapping,
    int64_t T, const float* rms_w, double eps, const float* cos_sin, int64_t cs_rows,
    int64_t cs_stride, uint8_t* k_cache, int64_t kv_bs, int64_t kv_stride0, int64_t n_kv_blocks,
    const int32_t* kv_slot_mapping, double* out_compressed, double* out_absnorm,
    double* out_normed, int32_t* out_status, int64_t t_lo, int64_t t_hi, int nthreads) {
  return oracle_compress_store(128, 0, HEAD, state, n_state_blocks, state_bs, s0, s1, block_table,
                               bt_rows, bt_cols, bt_stride, token_to_req, positions, slot_mapping,
                               T, rms_w, eps, cos_sin, cs_rows, cs_stride, k_cache, kv_bs,
                               kv_stride0, n_kv_blocks, kv_slot_mapping, out_compressed,
                               out_absnorm, out_normed, out_status, t_lo, t_hi, nthreads);
}

/* Array forms of the format helpers, for exhaustive tests. */
void oracle_bf16_bits_array(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_bits(x[i]);
}
void oracle_e4m3_code_array(const double* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_code(x[i]);
}
void oracle_ue8m0_exponent_array(const double* absmax, int32_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_ue8m0_exponent(absmax[i]);
}
void oracle_e2m1_code_array(const double* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_code(x[i]);
}
void oracle_mxfp4_exponent_array(const double* absmax, int32_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_mxfp4_exponent(absmax[i]);
}
