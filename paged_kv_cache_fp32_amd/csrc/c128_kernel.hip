// C128 compress-store kernel for MI355X (gfx950, wave64): the single pass.
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
//
// The fan-out (small batches) and compacted (varlen batches) schedules of the same computation
// are in c128_schedules.hip; the helpers both use are in c128_device.h.

#include "c128_device.h"
#include "c128_launch.h"

namespace dsv4 {
namespace {

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

  // ---- gate (all values wave-uniform; the whole workgroup takes one path).  The request id
  // does not depend on the gate, so it is loaded with the position and the slot: one dependent
  // round trip less before the block ids.  Its sign test joins the gate's own tests in one
  // branch; with the gate branching first, the compiler sinks the request load below it, into
  // a round trip of its own.
  const int32_t pos = p.positions[t];
  const int32_t slot = p.slot_mapping[t];
  const int32_t req = p.token_to_req[t];
  // Without the pooled-vector output a token with no kv slot writes nothing, so its kv slot is
  // loaded here too and joins the gate: no work for such a token, and no round trip for the
  // slot (and the kernel-argument line that holds its pointer) before the insert.
  const int32_t kv_slot = kDebug ? 0 : p.kv_slot_mapping[t];
  if ((slot < 0) | (pos < 0) | ((pos & (kRatio - 1)) != kRatio - 1) | (req < 0) | (kv_slot < 0))
    return;
  const int32_t win = pos >> 7;  // window rows 128*win .. 128*win + 127
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
  // The RoPE lanes' cos/sin pairs go out with rms_w (one round trip for both); every lane loads
  // a valid pair (lane & 15) and only lanes 48..63 of the second wave use it.  The empty asm
  // consumes them here: the compiler would otherwise sink the loads into the RoPE branch, which
  // runs after the quantised stores, into a round trip of their own.
  const int j = lane & 15;
  const float* cs = p.cos_sin + static_cast<int64_t>(rope_row) * p.cs_stride;
  const float c0 = cs[2 * j], c1 = cs[2 * j + 1];
  const float s0r = cs[kRope / 2 + 2 * j], s1r = cs[kRope / 2 + 2 * j + 1];
  asm volatile("" ::"v"(c0), "v"(c1), "v"(s0r), "v"(s1r));
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

  const int32_t kv = kDebug ? p.kv_slot_mapping[t] : kv_slot;
  if (kv < 0 || kv >= p.n_kv_slots) return;
  const int32_t kb = kv / p.kv_bs;
  const int32_t ko = kv - kb * p.kv_bs;
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
    // GPT-J RoPE: this lane (j = lane - 48) holds pairs m0 = 2j and m0 + 1 (dims 448 + 4j .. + 3)
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
  if (p.num_tokens >= kStagedMinTokens) return launch_c128_staged(p, stream);
  const dim3 grid(static_cast<unsigned>(p.num_tokens));
  const dim3 block(128 * kRowGroups);
  if (p.compressed_out)
    return launch_kernel(c128_compress_store_kernel<kRowGroups, kStageRows, kWavesPerSimd, true>,
                         grid, block, stream, p);
  return launch_kernel(c128_compress_store_kernel<kRowGroups, kStageRows, kWavesPerSimd, false>,
                       grid, block, stream, p);
}

hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  return launch_kernel(e4m3_encode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), stream,
                       in, out, n);
}

}  // namespace dsv4
