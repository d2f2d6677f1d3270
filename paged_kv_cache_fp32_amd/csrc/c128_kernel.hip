// C128 compress-store kernel for MI355X (gfx950, wave64).
//
// One workgroup per token.  What it computes follows the DeepSeek-V4
// sparse-attention fused kernel on the vLLM "fused_compress_quant_cache" API
// page (gate, window gather, per-column softmax pooling, RMSNorm, UE8M0/E4M3
// quantisation of the 448 nope dims, GPT-J RoPE of the 64 rope dims, paged
// insert).  How it computes it is specific to this chip:
//
//  * Column ownership.  A state row is 4 KiB: kv[0:512] | score[512:1024].
//    Lane l of a "column half" wave owns the 16-byte kv vector of columns
//    256*half + 4l .. +3 and the matching score vector 2 KiB further on, so
//    every wave-wide load is 1 KiB contiguous (fully coalesced).
//  * Row split.  The workgroup has 2*RG waves: the two column halves times
//    RG row groups; a row group streams 16/RG of the window's 16 state
//    blocks.  The window's 16 block ids are contiguous in the block table,
//    read once with wave-uniform (scalar) loads: no per-row table lookup.
//    State loads carry the non-temporal hint: the stream is read once.
//  * Online softmax in registers.  Rows are consumed in chunks of 4 with
//    the next chunk's loads already in flight; per column a lane keeps the
//    running max (in log2 units), the running sum of weights and the running
//    weighted sum, rescaled with exp2 when the max grows.
//  * Cross-wave merge through LDS (RG partial states per column), then the
//    fused epilogue on the 128 lanes of row group 0: RMSNorm sum of squares
//    by a wave reduction plus a 2-entry LDS exchange; one 64-column
//    quantisation block is exactly 16 lanes, so its absmax is a 4-step
//    in-group shuffle; the UE8M0 exponent comes from the bits of the fp32
//    product (exact ceil(log2)); codes use gfx950's OCP E4M3FN conversion;
//    RoPE lanes (columns 448..511) each rotate two pairs and store 8 bytes.
//
// This is an HBM-bound gather-reduce (about 0.6 flop per byte), so there is
// no MFMA: the work is dominated by streaming 512 KiB of state per token.

#include "c128_params.h"

namespace dsv4 {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFp8Max = 448.0f;
constexpr float kInvFp8Max = 1.0f / 448.0f;  // fl32(1/448), as the page's fp32 multiply uses
constexpr float kAbsmaxFloor = 1e-4f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int C>
__device__ __forceinline__ float lane_of(const float4& v) {
  if constexpr (C == 0) return v.x;
  else if constexpr (C == 1) return v.y;
  else if constexpr (C == 2) return v.z;
  else return v.w;
}

// Clamp to the E4M3FN range and convert four fp32 values to OCP FP8 E4M3FN
// (round to nearest even) with gfx950's packed conversion; byte k of the
// result is the code of the k-th argument.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = __builtin_fminf(__builtin_fmaxf(a, -kFp8Max), kFp8Max);
  b = __builtin_fminf(__builtin_fmaxf(b, -kFp8Max), kFp8Max);
  c = __builtin_fminf(__builtin_fmaxf(c, -kFp8Max), kFp8Max);
  d = __builtin_fminf(__builtin_fmaxf(d, -kFp8Max), kFp8Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)));
}

__device__ __forceinline__ float bf16_round(float x) {
  return __uint_as_float(bf16_bits(x) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Max over the 16-lane group holding one 64-column quantisation block.
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off));
  return v;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// State rows are read exactly once per call: load them with the non-temporal hint
// (global_load_dwordx4 ... nt) so the stream does not allocate in L2 / MALL.  On the
// 16-block window gather this lifts the attainable read rate from about 6.2 to 7.0 TB/s.
__device__ __forceinline__ float4 load_stream(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// CH rows starting at the wave-uniform row pointer `row` (SGPRs); the lane adds only its
// 32-bit column offset, so each load is the saddr + voffset form with no per-row VGPR address.
template <int CH>
__device__ __forceinline__ void load_rows(float4 (&kv)[CH], float4 (&sc)[CH], const float* row,
                                          int64_t s1, uint32_t col) {
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const float* rp = row + r * s1;
    kv[r] = load_stream(rp + col);
    sc[r] = load_stream(rp + kHead + col);
  }
}

// Online softmax update of one column with CH rows.
template <int C, bool kFirst, int CH>
__device__ __forceinline__ void update_column(const float4 (&kv)[CH], const float4 (&sc)[CH],
                                              float& ml, float& l, float& acc) {
  float s[CH];
#pragma unroll
  for (int r = 0; r < CH; ++r) s[r] = lane_of<C>(sc[r]);
  float cm = s[0];
#pragma unroll
  for (int r = 1; r < CH; ++r) cm = __builtin_fmaxf(cm, s[r]);
  cm *= kLog2e;
  const float mn = kFirst ? cm : __builtin_fmaxf(ml, cm);
  float psum = 0.0f, a = 0.0f;
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const float pr = exp2_fast(__builtin_fmaf(s[r], kLog2e, -mn));
    psum += pr;
    a = __builtin_fmaf(pr, lane_of<C>(kv[r]), a);
  }
  if (kFirst) {
    l = psum;
    acc = a;
  } else {
    const float scale = exp2_fast(ml - mn);
    l = __builtin_fmaf(l, scale, psum);
    acc = __builtin_fmaf(acc, scale, a);
  }
  ml = mn;
}

template <bool kFirst, int CH>
__device__ __forceinline__ void update(const float4 (&kv)[CH], const float4 (&sc)[CH],
                                       float (&ml)[4], float (&l)[4], float (&acc)[4]) {
  update_column<0, kFirst, CH>(kv, sc, ml[0], l[0], acc[0]);
  update_column<1, kFirst, CH>(kv, sc, ml[1], l[1], acc[1]);
  update_column<2, kFirst, CH>(kv, sc, ml[2], l[2], acc[2]);
  update_column<3, kFirst, CH>(kv, sc, ml[3], l[3], acc[3]);
}

// RG: row groups (the workgroup has 2*RG waves); CH: rows per pipeline stage; WPE: waves per
// SIMD the register allocation must allow (it bounds the VGPRs, hence the loads in flight).
template <int RG, int CH, int WPE, bool kDebug>
__global__ void __launch_bounds__(128 * RG) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
c128_compress_store_kernel(const C128Params p) {
  static_assert(kWindowBlocks % RG == 0, "row groups must split the 16 window blocks");
  static_assert(kStateBlock % CH == 0, "a stage must not straddle two state blocks");
  constexpr int NB = kWindowBlocks / RG;                 // state blocks per wave
  constexpr int NCH = NB * kStateBlock / CH;             // stages per wave (even)
  constexpr int kStagesPerBlock = kStateBlock / CH;
  static_assert(NCH % 2 == 0, "ping-pong needs an even chunk count");

  __shared__ float4 lds_ml[RG][2][64];
  __shared__ float4 lds_l[RG][2][64];
  __shared__ float4 lds_acc[RG][2][64];
  __shared__ float lds_ss[2];

  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave & 1;
  const int rg = wave >> 1;

  // ---- gate (all values wave-uniform; the whole workgroup takes one path)
  const int32_t pos = p.positions[t];
  const int32_t slot = p.slot_mapping[t];
  if (slot < 0 || pos < 0 || (pos & (kRatio - 1)) != kRatio - 1) return;
  const int32_t win = pos >> 7;  // window rows 128*win .. 128*win + 127
  const int32_t req = p.token_to_req[t];
  if (req < 0 || req >= p.bt_rows ||
      static_cast<int64_t>(win + 1) * kWindowBlocks > p.bt_cols)
    return;
  const int32_t rope_row = win * kRatio;  // (pos // 128) * 128
  if (rope_row >= p.cs_rows) return;
  const int32_t* bt =
      p.block_table + static_cast<int64_t>(req) * p.bt_stride +
      static_cast<int64_t>(win) * kWindowBlocks;
  bool ok = true;
#pragma unroll
  for (int i = 0; i < kWindowBlocks; ++i)
    ok &= static_cast<uint32_t>(bt[i]) < static_cast<uint32_t>(p.n_state_blocks);
  if (!ok) return;

  // ---- stream this wave's NB blocks x 8 rows, 4 rows per stage
  const int col = half * 256 + lane * 4;
  const uint32_t ucol = static_cast<uint32_t>(col);
  const int32_t* mybt = bt + rg * NB;
  const int64_t s0 = p.s0, s1 = p.s1;
  auto rowptr = [&](int ch) {  // wave-uniform
    return p.state + static_cast<int64_t>(mybt[ch / kStagesPerBlock]) * s0 +
           static_cast<int64_t>((ch % kStagesPerBlock) * CH) * s1;
  };

  float ml[4], l[4], acc[4];
  float4 kvA[CH], scA[CH], kvB[CH], scB[CH];
  load_rows<CH>(kvA, scA, rowptr(0), s1, ucol);
#pragma unroll
  for (int ch = 0; ch < NCH; ch += 2) {
    load_rows<CH>(kvB, scB, rowptr(ch + 1), s1, ucol);
    if (ch == 0)
      update<true, CH>(kvA, scA, ml, l, acc);
    else
      update<false, CH>(kvA, scA, ml, l, acc);
    if (ch + 2 < NCH) load_rows<CH>(kvA, scA, rowptr(ch + 2), s1, ucol);
    update<false, CH>(kvB, scB, ml, l, acc);
  }

  // ---- merge the RG row groups of each column half
  if constexpr (RG > 1) {
    lds_ml[rg][half][lane] = make_float4(ml[0], ml[1], ml[2], ml[3]);
    lds_l[rg][half][lane] = make_float4(l[0], l[1], l[2], l[3]);
    lds_acc[rg][half][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
  }
  float c[4] = {0.f, 0.f, 0.f, 0.f};
  if (rg == 0) {
    if constexpr (RG > 1) {
      // fold the other row groups into this wave's (m, l, acc) one at a time
#pragma unroll
      for (int g = 1; g < RG; ++g) {
        const float4 gm = lds_ml[g][half][lane];
        const float4 gl = lds_l[g][half][lane];
        const float4 ga = lds_acc[g][half][lane];
        const float om[4] = {gm.x, gm.y, gm.z, gm.w};
        const float ol[4] = {gl.x, gl.y, gl.z, gl.w};
        const float oa[4] = {ga.x, ga.y, ga.z, ga.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float M = __builtin_fmaxf(ml[k], om[k]);
          const float fs = exp2_fast(ml[k] - M), fo = exp2_fast(om[k] - M);
          l[k] = __builtin_fmaf(l[k], fs, ol[k] * fo);
          acc[k] = __builtin_fmaf(acc[k], fs, oa[k] * fo);
          ml[k] = M;
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = acc[k] / l[k];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = acc[k] / l[k];
    }
    // RMSNorm sum of squares: this lane's 4 columns, then the wave
    float ss = c[0] * c[0] + c[1] * c[1] + c[2] * c[2] + c[3] * c[3];
    ss = wave_sum(ss);
    if (lane == 0) lds_ss[half] = ss;
  }
  __syncthreads();
  if (rg != 0) return;

  // ---- fused epilogue on the 128 lanes of row group 0
  const float var = (lds_ss[0] + lds_ss[1]) * (1.0f / kHead);
  const float rrms = 1.0f / __builtin_sqrtf(var + p.eps);
  const float4 w = *reinterpret_cast<const float4*>(p.rms_w + col);
  float n[4] = {c[0] * rrms * w.x, c[1] * rrms * w.y, c[2] * rrms * w.z, c[3] * rrms * w.w};

  if constexpr (kDebug)
    *reinterpret_cast<float4*>(p.compressed_out + static_cast<int64_t>(t) * kHead + col) =
        make_float4(c[0], c[1], c[2], c[3]);

  // per-64 absmax of the bf16-rounded values (every lane joins the shuffles)
  float u[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] = bf16_round(n[k]);
  float amax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(u[0]), __builtin_fabsf(u[1])),
                               __builtin_fmaxf(__builtin_fabsf(u[2]), __builtin_fabsf(u[3])));
  amax = group16_max(amax);

  const int32_t kv_slot = p.kv_slot_mapping[t];
  if (kv_slot < 0 || kv_slot >= p.n_kv_slots) return;
  const int32_t kb = kv_slot / p.kv_bs;
  const int32_t ko = kv_slot - kb * p.kv_bs;
  uint8_t* blockp = p.k_cache + static_cast<int64_t>(kb) * p.kc_stride0;
  uint8_t* rec = blockp + static_cast<int64_t>(ko) * kRecordBytes;
  uint8_t* scl = blockp + static_cast<int64_t>(p.kv_bs) * kRecordBytes +
                 static_cast<int64_t>(ko) * kScaleBytes;

  const bool rope_lane = (half == 1) && (lane >= 48);
  if (!rope_lane) {
    // UE8M0 exponent: exact ceil(log2(raw)) from the fp32 bits of the product
    const float raw = __builtin_fmaxf(amax, kAbsmaxFloor) * kInvFp8Max;
    const uint32_t rb = __float_as_uint(raw);
    const int e = static_cast<int>((rb >> 23) & 0xffu) - 127 + ((rb & 0x7fffffu) != 0u);
    const float inv_scale = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);  // 2^-e
    const uint32_t codes = e4m3x4(u[0] * inv_scale, u[1] * inv_scale, u[2] * inv_scale,
                                  u[3] * inv_scale);
    *reinterpret_cast<uint32_t*>(rec + col) = codes;
    if ((lane & 15) == 0) {
      const int byte = e + 127;
      scl[col >> 6] = static_cast<uint8_t>(byte < 0 ? 0 : (byte > 255 ? 255 : byte));
    }
  } else {
    // GPT-J RoPE: this lane holds pairs m0 = 2j and m0 + 1 (dims 448 + 4j .. + 3)
    const int j = lane - 48;
    const float* cs = p.cos_sin + static_cast<int64_t>(rope_row) * p.cs_stride;
    const float c0 = cs[2 * j], c1 = cs[2 * j + 1];
    const float s0r = cs[kRope / 2 + 2 * j], s1r = cs[kRope / 2 + 2 * j + 1];
    const float x0 = n[0] * c0 - n[1] * s0r;
    const float y0 = n[1] * c0 + n[0] * s0r;
    const float x1 = n[2] * c1 - n[3] * s1r;
    const float y1 = n[3] * c1 + n[2] * s1r;
    const uint32_t lo = bf16_bits(x0) | (bf16_bits(y0) << 16);
    const uint32_t hi = bf16_bits(x1) | (bf16_bits(y1) << 16);
    *reinterpret_cast<uint2*>(rec + kNope + 8 * j) = make_uint2(lo, hi);
    if (j == 0) scl[kNumQuant] = 0;  // pad byte
  }
}

// ---------------------------------------------------------------------------------------------
// Pieces of the two fan-out kernels (the single-pass kernel above keeps its own inline form,
// which the compiler schedules better for the large-batch stream).

// Gate of token t and its window, all wave-uniform: active iff the state slot is >= 0 and the
// position closes a window; then request, window columns, RoPE row and the 16 block ids must be
// in range (device-resident values the host cannot check), else the token is skipped.
struct Window {
  bool ok;
  int32_t rope_row;      // (pos // 128) * 128
  const int32_t* bt;     // the window's 16 block ids
};

__device__ __forceinline__ Window gate_and_window(const C128Params& p, int32_t t) {
  Window w{false, 0, nullptr};
  const int32_t pos = p.positions[t];
  const int32_t slot = p.slot_mapping[t];
  if (slot < 0 || pos < 0 || (pos & (kRatio - 1)) != kRatio - 1) return w;
  const int32_t win = pos >> 7;  // window rows 128*win .. 128*win + 127
  const int32_t req = p.token_to_req[t];
  if (req < 0 || req >= p.bt_rows || static_cast<int64_t>(win + 1) * kWindowBlocks > p.bt_cols)
    return w;
  w.rope_row = win * kRatio;
  if (w.rope_row >= p.cs_rows) return w;
  w.bt = p.block_table + static_cast<int64_t>(req) * p.bt_stride +
         static_cast<int64_t>(win) * kWindowBlocks;
  bool ok = true;
#pragma unroll
  for (int i = 0; i < kWindowBlocks; ++i)
    ok &= static_cast<uint32_t>(w.bt[i]) < static_cast<uint32_t>(p.n_state_blocks);
  w.ok = ok;
  return w;
}

// Stream NBW state blocks (ids mybt[0..NBW)) x 8 rows, CH rows per stage, into this lane's
// online-softmax state (m in log2 units, l, acc) for its 4 columns.
template <int NBW, int CH>
__device__ __forceinline__ void stream_blocks(const C128Params& p, const int32_t* mybt,
                                              uint32_t ucol, float (&ml)[4], float (&l)[4],
                                              float (&acc)[4]) {
  constexpr int kStagesPerBlock = kStateBlock / CH;
  constexpr int NCH = NBW * kStagesPerBlock;  // stages (even)
  static_assert(kStateBlock % CH == 0, "a stage must not straddle two state blocks");
  static_assert(NCH % 2 == 0, "ping-pong needs an even stage count");
  const int64_t s0 = p.s0, s1 = p.s1;
  auto rowptr = [&](int ch) {  // wave-uniform
    return p.state + static_cast<int64_t>(mybt[ch / kStagesPerBlock]) * s0 +
           static_cast<int64_t>((ch % kStagesPerBlock) * CH) * s1;
  };
  float4 kvA[CH], scA[CH], kvB[CH], scB[CH];
  load_rows<CH>(kvA, scA, rowptr(0), s1, ucol);
#pragma unroll
  for (int ch = 0; ch < NCH; ch += 2) {
    load_rows<CH>(kvB, scB, rowptr(ch + 1), s1, ucol);
    if (ch == 0)
      update<true, CH>(kvA, scA, ml, l, acc);
    else
      update<false, CH>(kvA, scA, ml, l, acc);
    if (ch + 2 < NCH) load_rows<CH>(kvA, scA, rowptr(ch + 2), s1, ucol);
    update<false, CH>(kvB, scB, ml, l, acc);
  }
}

// Fold another partial (m, l, acc) of the same 4 columns into this one.
__device__ __forceinline__ void fold(float (&ml)[4], float (&l)[4], float (&acc)[4],
                                     const float4& gm, const float4& gl, const float4& ga) {
  const float om[4] = {gm.x, gm.y, gm.z, gm.w};
  const float ol[4] = {gl.x, gl.y, gl.z, gl.w};
  const float oa[4] = {ga.x, ga.y, ga.z, ga.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float M = __builtin_fmaxf(ml[k], om[k]);
    const float fs = exp2_fast(ml[k] - M), fo = exp2_fast(om[k] - M);
    l[k] = __builtin_fmaf(l[k], fs, ol[k] * fo);
    acc[k] = __builtin_fmaf(acc[k], fs, oa[k] * fo);
    ml[k] = M;
  }
}

// Merge the RG row groups of each column half through LDS: on return the rg == 0 waves hold
// the merged state.  Every wave of the workgroup must call it (it contains a barrier).
template <int RG>
__device__ __forceinline__ void merge_row_groups(float4 (&lds_ml)[RG][2][64],
                                                 float4 (&lds_l)[RG][2][64],
                                                 float4 (&lds_acc)[RG][2][64], int rg, int half,
                                                 int lane, float (&ml)[4], float (&l)[4],
                                                 float (&acc)[4]) {
  if constexpr (RG > 1) {
    lds_ml[rg][half][lane] = make_float4(ml[0], ml[1], ml[2], ml[3]);
    lds_l[rg][half][lane] = make_float4(l[0], l[1], l[2], l[3]);
    lds_acc[rg][half][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (rg == 0) {
#pragma unroll
      for (int g = 1; g < RG; ++g)
        fold(ml, l, acc, lds_ml[g][half][lane], lds_l[g][half][lane], lds_acc[g][half][lane]);
    }
  }
}

// Fused epilogue of token t on 128 lanes (2 waves, one per column half; 4 columns per lane):
// RMSNorm, bf16 round trip, per-64 absmax -> UE8M0 exponent -> E4M3FN codes, GPT-J RoPE ->
// bf16, paged insert.  sumsq is the sum of squares of all 512 pooled values.
template <bool kDebug>
__device__ __forceinline__ void epilogue(const C128Params& p, int32_t t, int32_t rope_row,
                                         const float (&c)[4], int half, int lane, int col,
                                         float sumsq) {
  const float var = sumsq * (1.0f / kHead);
  const float rrms = 1.0f / __builtin_sqrtf(var + p.eps);
  const float4 w = *reinterpret_cast<const float4*>(p.rms_w + col);
  float n[4] = {c[0] * rrms * w.x, c[1] * rrms * w.y, c[2] * rrms * w.z, c[3] * rrms * w.w};

  if constexpr (kDebug)
    *reinterpret_cast<float4*>(p.compressed_out + static_cast<int64_t>(t) * kHead + col) =
        make_float4(c[0], c[1], c[2], c[3]);

  // per-64 absmax of the bf16-rounded values (every lane joins the shuffles)
  float u[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] = bf16_round(n[k]);
  float amax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(u[0]), __builtin_fabsf(u[1])),
                               __builtin_fmaxf(__builtin_fabsf(u[2]), __builtin_fabsf(u[3])));
  amax = group16_max(amax);

  const int32_t kv_slot = p.kv_slot_mapping[t];
  if (kv_slot < 0 || kv_slot >= p.n_kv_slots) return;
  const int32_t kb = kv_slot / p.kv_bs;
  const int32_t ko = kv_slot - kb * p.kv_bs;
  uint8_t* blockp = p.k_cache + static_cast<int64_t>(kb) * p.kc_stride0;
  uint8_t* rec = blockp + static_cast<int64_t>(ko) * kRecordBytes;
  uint8_t* scl = blockp + static_cast<int64_t>(p.kv_bs) * kRecordBytes +
                 static_cast<int64_t>(ko) * kScaleBytes;

  const bool rope_lane = (half == 1) && (lane >= 48);
  if (!rope_lane) {
    // UE8M0 exponent: exact ceil(log2(raw)) from the fp32 bits of the product
    const float raw = __builtin_fmaxf(amax, kAbsmaxFloor) * kInvFp8Max;
    const uint32_t rb = __float_as_uint(raw);
    const int e = static_cast<int>((rb >> 23) & 0xffu) - 127 + ((rb & 0x7fffffu) != 0u);
    const float inv_scale = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);  // 2^-e
    const uint32_t codes = e4m3x4(u[0] * inv_scale, u[1] * inv_scale, u[2] * inv_scale,
                                  u[3] * inv_scale);
    *reinterpret_cast<uint32_t*>(rec + col) = codes;
    if ((lane & 15) == 0) {
      const int byte = e + 127;
      scl[col >> 6] = static_cast<uint8_t>(byte < 0 ? 0 : (byte > 255 ? 255 : byte));
    }
  } else {
    // GPT-J RoPE: this lane holds pairs m0 = 2j and m0 + 1 (dims 448 + 4j .. + 3)
    const int j = lane - 48;
    const float* cs = p.cos_sin + static_cast<int64_t>(rope_row) * p.cs_stride;
    const float c0 = cs[2 * j], c1 = cs[2 * j + 1];
    const float s0r = cs[kRope / 2 + 2 * j], s1r = cs[kRope / 2 + 2 * j + 1];
    const float x0 = n[0] * c0 - n[1] * s0r;
    const float y0 = n[1] * c0 + n[0] * s0r;
    const float x1 = n[2] * c1 - n[3] * s1r;
    const float y1 = n[3] * c1 + n[2] * s1r;
    const uint32_t lo = bf16_bits(x0) | (bf16_bits(y0) << 16);
    const uint32_t hi = bf16_bits(x1) | (bf16_bits(y1) << 16);
    *reinterpret_cast<uint2*>(rec + kNope + 8 * j) = make_uint2(lo, hi);
    if (j == 0) scl[kNumQuant] = 0;  // pad byte
  }
}

// c = acc / l, then the RMSNorm sum of squares over both column halves (one barrier), then the
// epilogue on the 128 lanes of the first two waves.  Every wave must call it.
template <bool kDebug>
__device__ __forceinline__ void finish_token(const C128Params& p, int32_t t, int32_t rope_row,
                                             bool epilogue_wave, int half, int lane, int col,
                                             const float (&l)[4], const float (&acc)[4],
                                             float* lds_ss) {
  float c[4] = {0.f, 0.f, 0.f, 0.f};
  if (epilogue_wave) {
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = acc[k] / l[k];
    float ss = c[0] * c[0] + c[1] * c[1] + c[2] * c[2] + c[3] * c[3];
    ss = wave_sum(ss);
    if (lane == 0) lds_ss[half] = ss;
  }
  __syncthreads();
  if (epilogue_wave) epilogue<kDebug>(p, t, rope_row, c, half, lane, col, lds_ss[0] + lds_ss[1]);
}

// ---------------------------------------------------------------------------------------------
// Fan-out for small batches: a token's 16 window blocks are split over S = RG*NBW... workgroups
// (grid = T x S).  Workgroup (t, s) streams window blocks s*RG*NBW .. (s+1)*RG*NBW - 1 and
// writes its merged partial state to the workspace:
//   ws[((t * S + s) * 3 + {0: m (log2 units), 1: l, 2: acc}) * 512 + column].
// The finish kernel then merges the S partials of each token and runs the epilogue.
template <int RG, int NBW, int CH>
__global__ void __launch_bounds__(128 * RG) c128_fanout_partial_kernel(const C128Params p,
                                                                     float* __restrict__ ws) {
  constexpr int kBlocksPerGroup = RG * NBW;
  static_assert(kWindowBlocks % kBlocksPerGroup == 0, "splits must divide the window");
  constexpr int S = kWindowBlocks / kBlocksPerGroup;

  __shared__ float4 lds_ml[RG][2][64];
  __shared__ float4 lds_l[RG][2][64];
  __shared__ float4 lds_acc[RG][2][64];

  const int32_t t = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave & 1;
  const int rg = wave >> 1;
  const int col = half * 256 + lane * 4;

  const Window win = gate_and_window(p, t);
  if (!win.ok) return;

  float ml[4], l[4], acc[4];
  stream_blocks<NBW, CH>(p, win.bt + s * kBlocksPerGroup + rg * NBW, static_cast<uint32_t>(col),
                         ml, l, acc);
  merge_row_groups<RG>(lds_ml, lds_l, lds_acc, rg, half, lane, ml, l, acc);
  if (rg == 0) {
    float* out = ws + (static_cast<int64_t>(t) * S + s) * (3 * kHead) + col;
    *reinterpret_cast<float4*>(out) = make_float4(ml[0], ml[1], ml[2], ml[3]);
    *reinterpret_cast<float4*>(out + kHead) = make_float4(l[0], l[1], l[2], l[3]);
    *reinterpret_cast<float4*>(out + 2 * kHead) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

// One workgroup of 128 lanes per token: merge the S partials, then the fused epilogue.
template <int S, bool kDebug>
__global__ void __launch_bounds__(128) c128_fanout_finish_kernel(const C128Params p,
                                                               const float* __restrict__ ws) {
  __shared__ float lds_ss[2];
  const int32_t t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = half * 256 + lane * 4;

  const Window win = gate_and_window(p, t);  // the same decision the partial kernel took
  if (!win.ok) return;

  const float* in = ws + static_cast<int64_t>(t) * S * (3 * kHead) + col;
  const float4 m0 = *reinterpret_cast<const float4*>(in);
  const float4 l0 = *reinterpret_cast<const float4*>(in + kHead);
  const float4 a0 = *reinterpret_cast<const float4*>(in + 2 * kHead);
  float ml[4] = {m0.x, m0.y, m0.z, m0.w};
  float l[4] = {l0.x, l0.y, l0.z, l0.w};
  float acc[4] = {a0.x, a0.y, a0.z, a0.w};
#pragma unroll
  for (int s = 1; s < S; ++s) {
    const float* q = in + s * (3 * kHead);
    fold(ml, l, acc, *reinterpret_cast<const float4*>(q),
         *reinterpret_cast<const float4*>(q + kHead),
         *reinterpret_cast<const float4*>(q + 2 * kHead));
  }
  finish_token<kDebug>(p, t, win.rope_row, true, half, lane, col, l, acc, lds_ss);
}

constexpr int kRowGroups = 4;  // 8 waves (512 lanes) per token
constexpr int kStageRows = 4;  // rows per pipeline stage
constexpr int kWavesPerSimd = 8;

// ---------------------------------------------------------------------------------------------
// Compacted schedule for long varlen batches (chunked prefill), where only about one token in
// 128 closes a window: a workgroup per token would spend most of the call dispatching
// workgroups that exit at the gate.  Two stream-ordered kernels, no atomics, deterministic:
//
//  1. c128_gate_scan_kernel: scan block b owns tokens [b*chunk, min(T, (b+1)*chunk)).  Its 256
//     lanes test the gate on 256 tokens at a time and write the tokens that pass, in token
//     order, to list[b*chunk + k], k < counts[b] (wave ballot, lane rank by mbcnt, per-wave
//     offsets through LDS).
//  2. c128_compacted_kernel: a persistent grid of single-pass-shaped workgroups.  Each builds
//     the exclusive prefix of counts[] in LDS and takes items blockIdx.x, blockIdx.x +
//     gridDim.x, ... of the compacted list; item i sits in the last scan block b with
//     prefix[b] <= i, at offset i - prefix[b].  A token then runs the full gate (its indices are
//     range-checked there), the window stream, the row-group merge and the fused epilogue.
constexpr int kScanThreads = 256;
constexpr int kMaxScanBlocks = 1024;
// The compacted kernel keeps loop-invariant values live across its tokens (about 108 VGPRs), so
// it runs 4 waves per SIMD: 2 workgroups of 8 waves per CU, a persistent grid of 512 for the
// 256 CUs.  Each wave still has a full pipeline stage of loads in flight.
constexpr int kCompactedWavesPerSimd = 4;
constexpr int kCompactedGrid = 512;

__global__ void __launch_bounds__(kScanThreads) c128_gate_scan_kernel(
    const C128Params p, int32_t chunk, int32_t* __restrict__ counts, int32_t* __restrict__ list) {
  __shared__ int32_t wave_count[kScanThreads / 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t end = begin + chunk < p.num_tokens ? begin + chunk : p.num_tokens;
  int32_t found = 0;  // tokens of this scan block that passed so far (uniform)
  for (int64_t base = begin; base < end; base += kScanThreads) {
    const int64_t t = base + threadIdx.x;
    bool act = false;
    if (t < end) {
      const int32_t pos = p.positions[t];
      const int32_t slot = p.slot_mapping[t];
      act = slot >= 0 && pos >= 0 && (pos & (kRatio - 1)) == kRatio - 1;
    }
    const uint64_t mask = __builtin_amdgcn_ballot_w64(act);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(mask >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
    if (lane == 0) wave_count[wave] = __builtin_popcountll(mask);
    __syncthreads();
    int32_t off = found, sum = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int32_t c = wave_count[w];
      if (w < wave) off += c;
      sum += c;
    }
    if (act) list[begin + off + below] = static_cast<int32_t>(t);
    found += sum;
    __syncthreads();  // wave_count is rewritten in the next round
  }
  if (threadIdx.x == 0) counts[blockIdx.x] = found;
}

template <bool kDebug>
__global__ void __launch_bounds__(128 * kRowGroups)
    __attribute__((amdgpu_waves_per_eu(kCompactedWavesPerSimd, kCompactedWavesPerSimd)))
    c128_compacted_kernel(const C128Params p, const int32_t* __restrict__ counts,
                          const int32_t* __restrict__ list, int32_t chunk, int32_t nblocks) {
  constexpr int RG = kRowGroups;
  constexpr int NBW = kWindowBlocks / RG;
  constexpr int kPerLane = kMaxScanBlocks / 64;

  __shared__ int32_t lds_prefix[kMaxScanBlocks];
  __shared__ int32_t lds_total;
  __shared__ float4 lds_ml[RG][2][64];
  __shared__ float4 lds_l[RG][2][64];
  __shared__ float4 lds_acc[RG][2][64];
  __shared__ float lds_ss[2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave & 1;
  const int rg = wave >> 1;
  const int col = half * 256 + lane * 4;

  // exclusive prefix of the scan-block counts: lane l of wave 0 owns blocks 16l .. 16l + 15
  if (wave == 0) {
    int32_t v[kPerLane];
    int32_t own = 0;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      const int b = lane * kPerLane + k;
      v[k] = b < nblocks ? counts[b] : 0;
      own += v[k];
    }
    int32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int32_t run = incl - own;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      const int b = lane * kPerLane + k;
      if (b < nblocks) lds_prefix[b] = run;
      run += v[k];
    }
    if (lane == 63) lds_total = incl;
  }
  __syncthreads();
  const int64_t total = __builtin_amdgcn_readfirstlane(lds_total);

  for (int64_t i = blockIdx.x; i < total; i += gridDim.x) {
    int lo = 0, hi = nblocks - 1;  // last b with prefix[b] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(lds_prefix[mid]) <= i)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int64_t at = static_cast<int64_t>(lo) * chunk +
                       (i - __builtin_amdgcn_readfirstlane(lds_prefix[lo]));
    const int32_t t = __builtin_amdgcn_readfirstlane(list[at]);
    const Window win = gate_and_window(p, t);
    if (win.ok) {
      float ml[4], l[4], acc[4];
      stream_blocks<NBW, kStageRows>(p, win.bt + rg * NBW, static_cast<uint32_t>(col), ml, l,
                                     acc);
      merge_row_groups<RG>(lds_ml, lds_l, lds_acc, rg, half, lane, ml, l, acc);
      finish_token<kDebug>(p, t, win.rope_row, rg == 0, half, lane, col, l, acc, lds_ss);
    }
    __syncthreads();  // LDS is reused by the next token
  }
}

__global__ void __launch_bounds__(256) e4m3_encode_kernel(const float* in, uint8_t* out,
                                                          int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  float v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = (i + k < n) ? in[i + k] : 0.0f;
  const uint32_t w = e4m3x4(v[0], v[1], v[2], v[3]);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (i + k < n) out[i + k] = static_cast<uint8_t>(w >> (8 * k));
}


}  // namespace

hipError_t launch_c128_compress_store(const C128Params& p, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.num_tokens));
  const dim3 block(128 * kRowGroups);
  if (p.compressed_out)
    c128_compress_store_kernel<kRowGroups, kStageRows, kWavesPerSimd, true>
        <<<grid, block, 0, stream>>>(p);
  else
    c128_compress_store_kernel<kRowGroups, kStageRows, kWavesPerSimd, false>
        <<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

namespace {

// Fan-out shapes: S splits of the 16 window blocks, each streamed by RG row groups of NBW blocks.
template <int RG, int NBW>
hipError_t launch_fanout(const C128Params& p, float* ws, hipStream_t stream) {
  constexpr int S = kWindowBlocks / (RG * NBW);
  const dim3 grid1(static_cast<unsigned>(p.num_tokens), S);
  c128_fanout_partial_kernel<RG, NBW, kStageRows><<<grid1, dim3(128 * RG), 0, stream>>>(p, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid2(static_cast<unsigned>(p.num_tokens));
  if (p.compressed_out)
    c128_fanout_finish_kernel<S, true><<<grid2, dim3(128), 0, stream>>>(p, ws);
  else
    c128_fanout_finish_kernel<S, false><<<grid2, dim3(128), 0, stream>>>(p, ws);
  return hipGetLastError();
}

}  // namespace

int fanout_auto_splits(int64_t num_tokens) {
  // Measured on MI355X with the window sets rotated (cold HBM): 8 splits are fastest up to 16
  // tokens, 4 up to 64; from about 100 tokens on the single pass already has enough
  // workgroups and the extra partial-state traffic and second launch make the fan-out slower.
  if (num_tokens <= 0 || num_tokens > 64) return 1;
  return num_tokens <= 16 ? 8 : 4;
}

size_t fanout_workspace_bytes(int64_t num_tokens, int splits) {
  if (splits <= 1 || num_tokens <= 0) return 0;
  return static_cast<size_t>(num_tokens) * static_cast<size_t>(splits) * 3 * kHead * sizeof(float);
}

hipError_t launch_c128_fanout(const C128Params& p, float* ws, int splits, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  switch (splits) {
    case 1:
      return launch_c128_compress_store(p, stream);
    case 2:
      return launch_fanout<4, 2>(p, ws, stream);
    case 4:
      return launch_fanout<4, 1>(p, ws, stream);
    case 8:
      return launch_fanout<2, 1>(p, ws, stream);
    case 16:
      return launch_fanout<1, 1>(p, ws, stream);
    default:
      return hipErrorInvalidValue;
  }
}

namespace {

// Scan blocks of a multiple of 256 tokens, at most kMaxScanBlocks of them.
void compacted_schedule(int64_t num_tokens, int32_t* chunk, int32_t* nblocks) {
  int64_t per = (num_tokens + kMaxScanBlocks - 1) / kMaxScanBlocks;
  if (per < 1) per = 1;
  const int64_t c = (per + kScanThreads - 1) / kScanThreads * kScanThreads;
  *chunk = static_cast<int32_t>(c);
  *nblocks = static_cast<int32_t>((num_tokens + c - 1) / c);
}

}  // namespace

size_t compacted_workspace_bytes(int64_t num_tokens) {
  if (num_tokens <= 0) return 0;
  const size_t ints = kMaxScanBlocks + static_cast<size_t>(num_tokens);
  return (ints * sizeof(int32_t) + 15) / 16 * 16;
}

hipError_t launch_c128_compacted(const C128Params& p, void* ws, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  int32_t chunk = 0, nblocks = 0;
  compacted_schedule(p.num_tokens, &chunk, &nblocks);
  int32_t* counts = static_cast<int32_t*>(ws);
  int32_t* list = counts + kMaxScanBlocks;
  c128_gate_scan_kernel<<<dim3(static_cast<unsigned>(nblocks)), dim3(kScanThreads), 0, stream>>>(
      p, chunk, counts, list);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned grid =
      static_cast<unsigned>(p.num_tokens < kCompactedGrid ? p.num_tokens : kCompactedGrid);
  if (p.compressed_out)
    c128_compacted_kernel<true><<<dim3(grid), dim3(128 * kRowGroups), 0, stream>>>(
        p, counts, list, chunk, nblocks);
  else
    c128_compacted_kernel<false><<<dim3(grid), dim3(128 * kRowGroups), 0, stream>>>(
        p, counts, list, chunk, nblocks);
  return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  e4m3_encode_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(in, out, n);
  return hipGetLastError();
}

}  // namespace dsv4
