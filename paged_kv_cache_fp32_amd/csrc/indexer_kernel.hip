// Indexer FP8 compress-store kernel for MI355X (gfx950, wave64).
//
// The DeepSeek-V4 indexer's compressor (vLLM "fused_compress_quant_cache" API page, kernel
// `_fused_kv_compress_norm_rope_insert_indexer_attn`), on the 8-row overlapping window of
// compress ratio 4: a token whose position closes a 4-row window (pos % 4 == 3, state slot
// >= 0) pools 8 state rows pos-7 .. pos per column (head 128; the previous window's rows
// contribute the first 128-column half of their kv and score parts, the current window's rows
// the second half; rows before position 0 take no part), applies RMSNorm, rotates dims 64..127
// as GPT-J pairs by table row (pos // 4) * 4, and only then quantises all 128 dims as one
// block: bf16 round trip, absmax (floor 1e-4), e = ceil(log2(absmax / 448)), E4M3FN codes of
// x * 2^-e, and the scale 2^e as one fp32.  A cache block holds bs records of 128 code bytes,
// then bs fp32 scales.
//
// The MXFP4 variant (same page, kernel `_fused_kv_compress_norm_rope_insert_indexer_mxfp4_attn`)
// shares everything up to the rotated, bf16-rounded values, then quantises four blocks of 32
// consecutive dims: e = ceil(log2(absmax / 6)) (absmax floored at 6 * 2^-126), E2M1 codes of
// x * 2^-e, two a byte with the even dim in the low nibble, and one UE8M0 byte e + 127 per
// block.  A cache block holds bs records of 64 bytes, then bs x 4 scale bytes.
//
// A state row is kv[0:256] | score[256:512]; a token reads 8 rows x 1 KiB = 8 KiB.
//
//  * One wave per token.  Lane l owns columns 2l, 2l+1 (8-byte vectors: each wave-wide load
//    is a 512-byte contiguous segment of a row), so lanes 32..63 hold exactly the 32 RoPE
//    pairs, and the RMSNorm sum and the quantisation absmax are single wave reductions.  An
//    MXFP4 block is the 16 lanes 16b..16b+15, and lane l packs byte l of the record.
//  * A wave takes 1 to 8 consecutive tokens (enough waves for 8 per SIMD first); their gate,
//    block ids and range checks are resolved up front, one lane per (token, window row).
//  * Records go to the wave's LDS stage and reach the cache after the wave's last state read,
//    so that the writes do not land in the middle of the HBM read stream.
//
// HBM-bound gather-reduce (about 0.6 flop per byte): no MFMA.

#include "c128_device.h"
#include "c128_launch.h"

namespace dsv4 {
namespace {

constexpr int kIdxHead = 128;
constexpr int kIdxNope = 64;                // dims before the RoPE dims
constexpr int kIdxRatio = 4;
constexpr int kIdxRows = 2 * kIdxRatio;     // previous window + current window
constexpr int kIdxScoreOffset = 2 * kIdxHead;
constexpr int kIdxRecord = 128;             // fp8 bytes per token
constexpr int kIdxScale = 4;                // one fp32 scale per token
constexpr int kIdxSlot = kIdxRecord + kIdxScale;
constexpr int kIdxWavesPerGroup = 4;
constexpr int kIdxMaxTokensPerWave = 8;     // 8 tokens x 8 window rows = the 64 lanes
constexpr int kIdxTargetWaves = 8192;       // 8 waves per SIMD on 256 CUs (57-59 VGPRs)
constexpr int kFp4Record = 64;              // E2M1 bytes per token, two dims a byte
constexpr int kFp4Scales = 4;               // one UE8M0 byte per 32-dim block
constexpr int kFp4Slot = kFp4Record + kFp4Scales;
constexpr float kFp4AbsmaxFloor = 0x1.8p-124f;  // 6 * 2^-126
constexpr float kInvFp4Max = 1.0f / 6.0f;       // fl32(1/6)

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float2 load_stream2(const float* p) {
  const f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
  return make_float2(v.x, v.y);
}

// E2M1 code of x in the low nibble: the nearest of the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6,
// ties to the even code, beyond 6 saturating to 6; bit 3 is the sign of x.  Each comparison
// is one midpoint between neighbouring magnitudes: strict where the code below it is the even
// one, inclusive where the code above it is.
__device__ __forceinline__ uint32_t e2m1(float x) {
  const float a = __builtin_fabsf(x);
  const uint32_t c = static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
                     static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
                     static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
                     static_cast<uint32_t>(a > 5.0f);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

template <bool kDebug, bool kFp4>
__global__ void __launch_bounds__(64 * kIdxWavesPerGroup)
    indexer_compress_store_kernel(const C128Params p, int32_t state_bs, int32_t state_bs_log2,
                                  int32_t tokens_per_wave) {
  constexpr int kSlot = kFp4 ? kFp4Slot : kIdxSlot;
  __shared__ __align__(16) uint8_t stage_all[kIdxWavesPerGroup][kIdxMaxTokensPerWave * kSlot];
  __shared__ int32_t slot_all[kIdxWavesPerGroup][kIdxMaxTokensPerWave];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* stage = stage_all[wave];
  int32_t* slot_of = slot_all[wave];
  const int64_t tbase = (static_cast<int64_t>(blockIdx.x) * kIdxWavesPerGroup + wave) *
                        tokens_per_wave;
  if (lane < kIdxMaxTokensPerWave) slot_of[lane] = -1;

  // ---- metadata, one lane per (token k, window row i); a token goes on only if all 8 of its
  // lanes pass.  Rows before position 0 (pos 3, i < 4) are not read.
  const int mk = lane >> 3, mi = lane & 7;
  const int64_t mt = tbase + mk;
  int32_t mpos = -1, mkv = -1;
  int64_t moff = 0;
  bool mok = false;
  if (mk < tokens_per_wave && mt < p.num_tokens) {
    // the request id and the kv slot are loaded with the gate's position and slot: the block
    // ids then wait for one round trip, not two
    mpos = p.positions[mt];
    const int32_t slot = p.slot_mapping[mt];
    const int32_t req = p.token_to_req[mt];
    const int32_t kvs = mi == 0 ? p.kv_slot_mapping[mt] : -1;
    if (slot >= 0 && mpos >= 0 && (mpos & (kIdxRatio - 1)) == kIdxRatio - 1) {
      mok = req >= 0 && req < p.bt_rows && mpos / state_bs < p.bt_cols &&
            (mpos & ~(kIdxRatio - 1)) < p.cs_rows;
      const int32_t q = mpos - (kIdxRows - 1) + mi;
      if (mok && q >= 0) {
        const int32_t bcol = state_bs_log2 >= 0 ? q >> state_bs_log2 : q / state_bs;
        const int32_t boff = q - bcol * state_bs;
        const int32_t b = p.block_table[static_cast<int64_t>(req) * p.bt_stride + bcol];
        mok = static_cast<uint32_t>(b) < static_cast<uint32_t>(p.n_state_blocks);
        moff = static_cast<int64_t>(b) * p.s0 + static_cast<int64_t>(boff) * p.s1 +
               (mi >= kIdxRatio ? kIdxHead : 0);
      }
      mkv = kvs;
    }
  }
  const uint64_t good = __builtin_amdgcn_ballot_w64(mok);

  const uint32_t col = static_cast<uint32_t>(lane) * 2;
  const float2 w = *reinterpret_cast<const float2*>(p.rms_w + col);
  const bool rope_lane = lane >= kIdxNope / 2;
  const int m = lane & 31;  // RoPE pair of lanes 32..63: dims 64 + 2m, 65 + 2m

  for (int k = 0; k < tokens_per_wave; ++k) {
    if (((good >> (8 * k)) & 0xffu) != 0xffu) continue;  // inactive or an index out of range
    const int32_t pos = __builtin_amdgcn_readlane(mpos, 8 * k);
    const int32_t kv_slot = __builtin_amdgcn_readlane(mkv, 8 * k);
    const float* rowp[kIdxRows];
#pragma unroll
    for (int i = 0; i < kIdxRows; ++i) {
      const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(moff), 8 * k + i);
      const uint32_t hi =
          __builtin_amdgcn_readlane(static_cast<uint32_t>(static_cast<uint64_t>(moff) >> 32),
                                    8 * k + i);
      rowp[i] = p.state + static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    }
    const float* cs = p.cos_sin + static_cast<int64_t>(pos & ~(kIdxRatio - 1)) * p.cs_stride;
    const float cosv = cs[m], sinv = cs[kRope / 2 + m];

    // ---- pool: 8 rows, or only the current window's 4 at position 3
    const int first = pos >= kIdxRows - 1 ? 0 : kIdxRatio;
    float2 kv[kIdxRows], sc[kIdxRows];
#pragma unroll
    for (int i = 0; i < kIdxRows; ++i) {
      if (i < first) continue;
      kv[i] = load_stream2(rowp[i] + col);
      sc[i] = load_stream2(rowp[i] + kIdxScoreOffset + col);
    }
    float mx = -__builtin_inff(), my = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kIdxRows; ++i) {
      if (i < first) continue;
      mx = __builtin_fmaxf(mx, sc[i].x * kLog2e);
      my = __builtin_fmaxf(my, sc[i].y * kLog2e);
    }
    float lx = 0.f, ly = 0.f, ax = 0.f, ay = 0.f;
#pragma unroll
    for (int i = 0; i < kIdxRows; ++i) {
      if (i < first) continue;
      const float px = exp2_fast(__builtin_fmaf(sc[i].x, kLog2e, -mx));
      const float py = exp2_fast(__builtin_fmaf(sc[i].y, kLog2e, -my));
      lx += px;
      ly += py;
      ax = __builtin_fmaf(px, kv[i].x, ax);
      ay = __builtin_fmaf(py, kv[i].y, ay);
    }
    const float c0 = ax / lx, c1 = ay / ly;

    // ---- RMSNorm over the 128 columns
    const float ss = wave_sum(__builtin_fmaf(c0, c0, c1 * c1));
    const float rrms = 1.0f / __builtin_sqrtf(ss * (1.0f / kIdxHead) + p.eps);
    const float n0 = c0 * rrms * w.x, n1 = c1 * rrms * w.y;
    if constexpr (kDebug)
      *reinterpret_cast<float2*>(p.compressed_out + (tbase + k) * kIdxHead + col) =
          make_float2(c0, c1);
    if (kv_slot < 0 || kv_slot >= p.n_kv_slots) continue;

    // ---- RoPE (lanes 32..63), then the quantisation
    const float r0 = rope_lane ? n0 * cosv - n1 * sinv : n0;
    const float r1 = rope_lane ? n1 * cosv + n0 * sinv : n1;
    const float u0 = bf16_round(r0), u1 = bf16_round(r1);
    if constexpr (kFp4) {
      // four 32-dim blocks of 16 lanes; lane l writes byte l, lane 16b the scale of block b
      const float amax = group16_max(__builtin_fmaxf(__builtin_fabsf(u0), __builtin_fabsf(u1)));
      const float raw = __builtin_fmaxf(amax, kFp4AbsmaxFloor) * kInvFp4Max;
      const uint32_t rb = __float_as_uint(raw);
      int e = static_cast<int>((rb >> 23) & 0xffu) - 127 + ((rb & 0x7fffffu) != 0u);
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
      const float inv = __builtin_ldexpf(1.0f, -e);
      uint8_t* rec = stage + k * kSlot;
      rec[lane] = static_cast<uint8_t>(e2m1(u0 * inv) | (e2m1(u1 * inv) << 4));
      if ((lane & 15) == 0) rec[kFp4Record + (lane >> 4)] = static_cast<uint8_t>(e + 127);
      if (lane == 0) slot_of[k] = kv_slot;
      continue;
    }
    const float amax = wave_max(__builtin_fmaxf(__builtin_fabsf(u0), __builtin_fabsf(u1)));
    const float raw = __builtin_fmaxf(amax, kAbsmaxFloor) * kInvFp8Max;
    const uint32_t rb = __float_as_uint(raw);
    const int e = static_cast<int>((rb >> 23) & 0xffu) - 127 + ((rb & 0x7fffffu) != 0u);
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);  // 2^-e
    const uint32_t codes = e4m3x4(u0 * inv, u1 * inv, 0.0f, 0.0f) & 0xffffu;
    uint8_t* rec = stage + k * kSlot;
    *reinterpret_cast<uint16_t*>(rec + col) = static_cast<uint16_t>(codes);
    if (lane == 0) {
      *reinterpret_cast<uint32_t*>(rec + kIdxRecord) = static_cast<uint32_t>(e + 127) << 23;
      slot_of[k] = kv_slot;
    }
  }

  // ---- insert every staged record after the wave's last state read (4-byte stores; records
  // and scales are 4-byte aligned)
  for (int k = 0; k < tokens_per_wave; ++k) {
    const int32_t kv_slot = slot_of[k];
    if (kv_slot < 0) continue;
    const int32_t kb = kv_slot / p.kv_bs;
    const int32_t ko = kv_slot - kb * p.kv_bs;
    uint8_t* blockp = p.k_cache + static_cast<int64_t>(kb) * p.kc_stride0;
    const uint8_t* rec = stage + k * kSlot;
    constexpr int kRec = kFp4 ? kFp4Record : kIdxRecord;  // data bytes; then 4 scale bytes
    if (lane < kRec / 4)
      *reinterpret_cast<uint32_t*>(blockp + static_cast<int64_t>(ko) * kRec + 4 * lane) =
          *reinterpret_cast<const uint32_t*>(rec + 4 * lane);
    else if (lane == kRec / 4)
      *reinterpret_cast<uint32_t*>(blockp + static_cast<int64_t>(p.kv_bs) * kRec +
                                   static_cast<int64_t>(ko) * 4) =
          *reinterpret_cast<const uint32_t*>(rec + kRec);
  }
}

__global__ void __launch_bounds__(256) e2m1_encode_kernel(const float* in, uint8_t* out,
                                                          int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = static_cast<uint8_t>(e2m1(in[i]));
}

int indexer_tokens_per_wave(int64_t num_tokens) {
  int64_t k = (num_tokens + kIdxTargetWaves - 1) / kIdxTargetWaves;
  return static_cast<int>(k < 1 ? 1 : (k > kIdxMaxTokensPerWave ? kIdxMaxTokensPerWave : k));
}

template <bool kFp4>
hipError_t launch_indexer(const C128Params& p, int32_t state_bs, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  const int32_t kpw = indexer_tokens_per_wave(p.num_tokens);
  const int64_t waves = (static_cast<int64_t>(p.num_tokens) + kpw - 1) / kpw;
  const int64_t groups = (waves + kIdxWavesPerGroup - 1) / kIdxWavesPerGroup;
  const dim3 grid(static_cast<unsigned>(groups));
  const dim3 block(64 * kIdxWavesPerGroup);
  const int32_t lg = (state_bs & (state_bs - 1)) == 0 ? __builtin_ctz(state_bs) : -1;
  if (p.compressed_out)
    return launch_kernel(indexer_compress_store_kernel<true, kFp4>, grid, block, stream, p,
                         state_bs, lg, kpw);
  return launch_kernel(indexer_compress_store_kernel<false, kFp4>, grid, block, stream, p,
                       state_bs, lg, kpw);
}

}  // namespace

hipError_t launch_indexer_compress_store(const C128Params& p, int32_t state_bs,
                                         hipStream_t stream) {
  return launch_indexer<false>(p, state_bs, stream);
}

hipError_t launch_indexer_mxfp4_compress_store(const C128Params& p, int32_t state_bs,
                                               hipStream_t stream) {
  return launch_indexer<true>(p, state_bs, stream);
}

hipError_t launch_e2m1_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  return launch_kernel(e2m1_encode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), stream,
                       in, out, n);
}

}  // namespace dsv4
