// C4 compress-store kernel for MI355X (gfx950, wave64).
//
// The DeepSeek-V4 C4 compressor: the sparse-attention fused kernel of the vLLM
// "fused_compress_quant_cache" API page run with compress ratio 4 and overlap 1.  A token
// whose position closes a 4-row window (pos % 4 == 3, state slot >= 0) pools 8 state rows,
// pos-7 .. pos: the previous window's 4 rows contribute the first 512-column half of their kv
// and score parts, the current window's 4 rows the second half, and rows before position 0
// take no part.  Then RMSNorm, the UE8M0/E4M3 quantisation of the 448 nope dims, GPT-J RoPE of
// the 64 rope dims at table row (pos // 4) * 4, and the paged insert, all as in the C128 path.
//
// A state row is kv[0:1024] | score[1024:2048] (2 x 512 each).  A token reads 8 rows x 4 KiB
// = 32 KiB, a sixteenth of a C128 token, so the whole token fits one wave:
//
//  * One wave per token, four tokens per workgroup; no LDS and no barrier.  Lane l owns
//    columns 4l .. 4l+3 ("v0") and 256 + 4l .. +3 ("v1"), so each wave-wide load is a 1 KiB
//    contiguous segment of a row.
//  * All loads of the window (up to 8 rows x 4 vectors, non-temporal) are issued before any
//    arithmetic; the per-column softmax is a plain max / exp2-sum over registers.
//  * Epilogue within the wave: RMSNorm by one wave reduction; a 64-column quant block is 16
//    lanes of v0 (blocks 0..3) or of v1 (blocks 4..6); lanes 48..63 hold the RoPE dims in v1.
//
// HBM-bound gather-reduce again (about 0.6 flop per byte): no MFMA.

#include "c128_device.h"
#include "c128_launch.h"

namespace dsv4 {
namespace {

constexpr int kC4Ratio = 4;
constexpr int kC4Rows = 2 * kC4Ratio;       // previous window + current window
constexpr int kC4ScoreOffset = 2 * kHead;   // score part of a row: 2 x 512 columns in
constexpr int kC4TokensPerGroup = 4;        // waves (tokens) per workgroup

// Per-column softmax-weighted sum over NR rows held in registers (scores scaled to log2).
template <int NR>
__device__ __forceinline__ float pool_column(const float (&s)[NR], const float (&kv)[NR]) {
  float m = s[0];
#pragma unroll
  for (int r = 1; r < NR; ++r) m = __builtin_fmaxf(m, s[r]);
  float l = 0.0f, a = 0.0f;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float p = exp2_fast(s[r] - m);
    l += p;
    a = __builtin_fmaf(p, kv[r], a);
  }
  return a / l;
}

// Load NR window rows (row pointers already offset to the row's kv half) and pool the lane's
// 8 columns into c[0..3] (v0) and c[4..7] (v1).
template <int NR>
__device__ __forceinline__ void pool_rows(const float* const (&rowp)[NR], uint32_t col,
                                          float (&c)[8]) {
  float4 kv0[NR], kv1[NR], sc0[NR], sc1[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    kv0[r] = load_stream(rowp[r] + col);
    kv1[r] = load_stream(rowp[r] + 256 + col);
    sc0[r] = load_stream(rowp[r] + kC4ScoreOffset + col);
    sc1[r] = load_stream(rowp[r] + kC4ScoreOffset + 256 + col);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float s[NR], v[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      s[r] = (k == 0 ? sc0[r].x : k == 1 ? sc0[r].y : k == 2 ? sc0[r].z : sc0[r].w) * kLog2e;
      v[r] = k == 0 ? kv0[r].x : k == 1 ? kv0[r].y : k == 2 ? kv0[r].z : kv0[r].w;
    }
    c[k] = pool_column<NR>(s, v);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      s[r] = (k == 0 ? sc1[r].x : k == 1 ? sc1[r].y : k == 2 ? sc1[r].z : sc1[r].w) * kLog2e;
      v[r] = k == 0 ? kv1[r].x : k == 1 ? kv1[r].y : k == 2 ? kv1[r].z : kv1[r].w;
    }
    c[4 + k] = pool_column<NR>(s, v);
  }
}

// UE8M0 exponent of a quant block from its absmax: exact ceil(log2(max(absmax, 1e-4) *
// fl32(1/448))) from the bits of the fp32 product.
__device__ __forceinline__ int ue8m0_exponent(float amax) {
  const float raw = __builtin_fmaxf(amax, kAbsmaxFloor) * kInvFp8Max;
  const uint32_t rb = __float_as_uint(raw);
  return static_cast<int>((rb >> 23) & 0xffu) - 127 + ((rb & 0x7fffffu) != 0u);
}

__device__ __forceinline__ uint32_t quant4(const float (&u)[8], int o, int e) {
  const float inv = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);  // 2^-e
  return e4m3x4(u[o] * inv, u[o + 1] * inv, u[o + 2] * inv, u[o + 3] * inv);
}

__device__ __forceinline__ uint8_t scale_byte(int e) {
  const int b = e + 127;
  return static_cast<uint8_t>(b < 0 ? 0 : (b > 255 ? 255 : b));
}

template <bool kDebug>
__global__ void __launch_bounds__(64 * kC4TokensPerGroup)
    c4_compress_store_kernel(const C128Params p, int32_t state_bs) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kC4TokensPerGroup + wave;
  if (t >= p.num_tokens) return;

  // ---- gate and window (wave-uniform); out-of-range device indices skip the token
  const int32_t pos = p.positions[t];
  const int32_t slot = p.slot_mapping[t];
  if (slot < 0 || pos < 0 || (pos & (kC4Ratio - 1)) != kC4Ratio - 1) return;
  const int32_t req = p.token_to_req[t];
  if (req < 0 || req >= p.bt_rows || pos / state_bs >= p.bt_cols) return;
  const int32_t rope_row = pos & ~(kC4Ratio - 1);  // (pos // 4) * 4
  if (rope_row >= p.cs_rows) return;
  const int32_t* bt = p.block_table + static_cast<int64_t>(req) * p.bt_stride;
  const int32_t start = pos - (kC4Rows - 1);
  const float* rowp[kC4Rows];
  bool ok = true;
#pragma unroll
  for (int i = 0; i < kC4Rows; ++i) {
    const int32_t q = start + i;
    rowp[i] = p.state;
    if (q < 0) continue;
    const int32_t b = bt[q / state_bs];
    ok &= static_cast<uint32_t>(b) < static_cast<uint32_t>(p.n_state_blocks);
    rowp[i] = p.state + static_cast<int64_t>(b) * p.s0 + static_cast<int64_t>(q % state_bs) * p.s1 +
              (i >= kC4Ratio ? kHead : 0);
  }
  if (!ok) return;

  // ---- pool: 8 rows, or only the current window's 4 when the previous one lies before 0
  const uint32_t col = static_cast<uint32_t>(lane) * 4;
  float c[8];
  if (start >= 0) {
    pool_rows<kC4Rows>(rowp, col, c);
  } else {
    const float* const cur[kC4Ratio] = {rowp[4], rowp[5], rowp[6], rowp[7]};
    pool_rows<kC4Ratio>(cur, col, c);
  }

  // ---- RMSNorm over the 512 columns (one wave)
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss = __builtin_fmaf(c[k], c[k], ss);
  ss = wave_sum(ss);
  const float rrms = 1.0f / __builtin_sqrtf(ss * (1.0f / kHead) + p.eps);
  const float4 w0 = *reinterpret_cast<const float4*>(p.rms_w + col);
  const float4 w1 = *reinterpret_cast<const float4*>(p.rms_w + 256 + col);
  const float n[8] = {c[0] * rrms * w0.x, c[1] * rrms * w0.y, c[2] * rrms * w0.z,
                      c[3] * rrms * w0.w, c[4] * rrms * w1.x, c[5] * rrms * w1.y,
                      c[6] * rrms * w1.z, c[7] * rrms * w1.w};
  if constexpr (kDebug) {
    float* out = p.compressed_out + t * kHead;
    *reinterpret_cast<float4*>(out + col) = make_float4(c[0], c[1], c[2], c[3]);
    *reinterpret_cast<float4*>(out + 256 + col) = make_float4(c[4], c[5], c[6], c[7]);
  }

  // ---- per-64 absmax of the bf16-rounded values (every lane joins both shuffles)
  float u[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) u[k] = bf16_round(n[k]);
  const float a0 = group16_max(__builtin_fmaxf(
      __builtin_fmaxf(__builtin_fabsf(u[0]), __builtin_fabsf(u[1])),
      __builtin_fmaxf(__builtin_fabsf(u[2]), __builtin_fabsf(u[3]))));
  const float a1 = group16_max(__builtin_fmaxf(
      __builtin_fmaxf(__builtin_fabsf(u[4]), __builtin_fabsf(u[5])),
      __builtin_fmaxf(__builtin_fabsf(u[6]), __builtin_fabsf(u[7]))));

  // ---- paged insert
  const int32_t kv_slot = p.kv_slot_mapping[t];
  if (kv_slot < 0 || kv_slot >= p.n_kv_slots) return;
  const int32_t kb = kv_slot / p.kv_bs;
  const int32_t ko = kv_slot - kb * p.kv_bs;
  uint8_t* blockp = p.k_cache + static_cast<int64_t>(kb) * p.kc_stride0;
  uint8_t* rec = blockp + static_cast<int64_t>(ko) * kRecordBytes;
  uint8_t* scl = blockp + static_cast<int64_t>(p.kv_bs) * kRecordBytes +
                 static_cast<int64_t>(ko) * kScaleBytes;
  const int group = lane >> 4;

  // v0: columns 0..255, quant blocks 0..3
  const int e0 = ue8m0_exponent(a0);
  *reinterpret_cast<uint32_t*>(rec + col) = quant4(u, 0, e0);
  if ((lane & 15) == 0) scl[group] = scale_byte(e0);

  if (lane < 48) {
    // v1: columns 256..447, quant blocks 4..6
    const int e1 = ue8m0_exponent(a1);
    *reinterpret_cast<uint32_t*>(rec + 256 + col) = quant4(u, 4, e1);
    if ((lane & 15) == 0) scl[4 + group] = scale_byte(e1);
  } else {
    // v1 of lanes 48..63: RoPE dims 448 + 4j .. +3, pairs 2j and 2j + 1
    const int j = lane - 48;
    const float* cs = p.cos_sin + static_cast<int64_t>(rope_row) * p.cs_stride;
    const float c0 = cs[2 * j], c1 = cs[2 * j + 1];
    const float s0 = cs[kRope / 2 + 2 * j], s1 = cs[kRope / 2 + 2 * j + 1];
    const float x0 = n[4] * c0 - n[5] * s0;
    const float y0 = n[5] * c0 + n[4] * s0;
    const float x1 = n[6] * c1 - n[7] * s1;
    const float y1 = n[7] * c1 + n[6] * s1;
    const uint32_t lo = bf16_bits(x0) | (bf16_bits(y0) << 16);
    const uint32_t hi = bf16_bits(x1) | (bf16_bits(y1) << 16);
    *reinterpret_cast<uint2*>(rec + kNope + 8 * j) = make_uint2(lo, hi);
    if (j == 0) scl[kNumQuant] = 0;  // pad byte
  }
}

}  // namespace

hipError_t launch_c4_compress_store(const C128Params& p, int32_t state_bs, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  const int64_t groups = (static_cast<int64_t>(p.num_tokens) + kC4TokensPerGroup - 1) /
                         kC4TokensPerGroup;
  const dim3 grid(static_cast<unsigned>(groups));
  const dim3 block(64 * kC4TokensPerGroup);
  if (p.compressed_out)
    c4_compress_store_kernel<true><<<grid, block, 0, stream>>>(p, state_bs);
  else
    c4_compress_store_kernel<false><<<grid, block, 0, stream>>>(p, state_bs);
  return hipGetLastError();
}

}  // namespace dsv4
