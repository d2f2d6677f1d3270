// Device helpers of the C128 compress-store kernels: fp8 / bf16 conversions, wave and 16-lane
// reductions, the non-temporal state-row loads and the per-column online-softmax update, plus
// the single pass's launch shape (the compacted schedule reuses it).
#pragma once

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

// Wave reductions with DPP lane moves instead of LDS-crossbar shuffles (ds_bpermute).  Lanes
// i ^ 1 and i ^ 2 are quad permutes; after them every quad holds one value, so the mirror within
// 8 lanes pairs each quad with its neighbour, and then the mirror within 16 lanes pairs the two
// half-rows.  The four 16-lane rows are combined through readlane.  Every lane gets the result;
// the whole wave must be active.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over the wave: quads, half-rows and rows by DPP, then (row0 + row1) + (row2 + row3).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xb1>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);  // row_half_mirror
  v += dpp_move<0x140>(v);  // row_mirror
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Max over each 16-lane row (a 64-column quantisation block of 4 columns a lane, or a 32-dim
// MXFP4 block of 2 a lane); exact in any order.
__device__ __forceinline__ float group16_max(float v) {
  v = __builtin_fmaxf(v, dpp_move<0xb1>(v));
  v = __builtin_fmaxf(v, dpp_move<0x4e>(v));
  v = __builtin_fmaxf(v, dpp_move<0x141>(v));
  return __builtin_fmaxf(v, dpp_move<0x140>(v));
}

// Max over the wave.
__device__ __forceinline__ float wave_max(float v) {
  v = group16_max(v);
  return __builtin_fmaxf(__builtin_fmaxf(lane_value(v, 0), lane_value(v, 16)),
                         __builtin_fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Loads that write LDS directly (global_load_lds_dword / _dwordx4): each active lane reads 4
// bytes, or 16 from a 16-byte aligned address, at g, and lane i's bytes land at lds + 4 * i or
// lds + 16 * i (lds wave-uniform).  No register holds the data, so inputs that are needed only
// at the end of a kernel can be fetched at its start at no register cost.  The compiler counts
// these loads like any other and waits for them before LDS reads of the same memory.
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void load_to_lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((global_void*)(const_cast<void*>(g)), (lds_void*)(lds), 4, 0, 0);
}
__device__ __forceinline__ void load_to_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((global_void*)(const_cast<void*>(g)), (lds_void*)(lds), 16, 0,
                                   0);
}

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
  // No contraction in here: the stage maximum cm = fl(max(s) * log2 e) must stay a rounded
  // product.  Every weight of the stage is exp2(s * log2 e - cm) with one shared cm, so the
  // rounding of cm cancels when the weights are normalised; a later stage rescales this one by
  // exp2(ml - mn) with ml == cm.  Under -ffp-contract=fast the compiler may fuse the multiply
  // into that subtraction, which then sees the exact product instead of cm, and the rounding of
  // cm (half an ulp of s * log2 e) stops cancelling between the stages.  The explicit fmaf
  // calls below stay fused.
#pragma clang fp contract(off)
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

constexpr int kRowGroups = 4;  // 8 waves (512 lanes) per token
constexpr int kStageRows = 4;  // rows per pipeline stage
constexpr int kWavesPerSimd = 8;

}  // namespace
}  // namespace dsv4
