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
// = 32 KiB, a sixteenth of a C128 token, so a token fits one wave:
//
//  * Lane l owns columns 4l .. 4l+3 ("v0") and 256 + 4l .. +3 ("v1"), so each wave-wide load
//    is a 1 KiB contiguous segment of a row.  All loads of a window (up to 8 rows x 4 vectors,
//    non-temporal) are issued before any arithmetic; the per-column softmax is a plain max /
//    exp2-sum over registers.  Waves stream independently; the only barriers are around the
//    workgroup's token list and before its record flush.
//  * Metadata is resolved 8 tokens at a time with one lane per (token, window row): gate,
//    request, block column, block id and range checks in two rounds of loads, so the token
//    loop only moves row offsets from lanes to scalars and streams.
//  * Small batches run 4-wave workgroups, each wave on 1 to 8 consecutive tokens (enough waves
//    for 2 per SIMD first).  From 8192 tokens, while one round covers the batch (up to 49,152
//    tokens), a workgroup is 12 waves (one per CU, 3 per SIMD) of up to 16 tokens each; it
//    gates all of its tokens first and deals the passing ones out to its waves in turn.
//  * Epilogue within the wave: RMSNorm by one wave reduction; a 64-column quant block is 16
//    lanes of v0 (blocks 0..3) or of v1 (blocks 4..6); lanes 48..63 hold the RoPE dims in v1.
//    Records go to the wave's LDS stage and reach the k_cache after the last state read of
//    every wave of the workgroup: measured on MI355X, the same 584-byte records stored token by
//    token cost about 12% of the call, and stored at the end of each wave about 8% (16384
//    tokens), because the writes land in the middle of the HBM read stream.  Holding a whole
//    CU's records to the end of its reads takes most of that back.
//
// HBM-bound gather-reduce again (about 0.6 flop per byte): no MFMA.

#include "c128_device.h"
#include "c128_launch.h"

namespace dsv4 {
namespace {

constexpr int kC4Ratio = 4;
constexpr int kC4Rows = 2 * kC4Ratio;       // previous window + current window
constexpr int kC4ScoreOffset = 2 * kHead;   // score part of a row: 2 x 512 columns in
constexpr int kC4NarrowWaves = 4;           // waves per workgroup, small batches
constexpr int kC4WideWaves = 12;            // waves per workgroup from kC4WideMinTokens on
constexpr int kC4WideMinTokens = 8192;
constexpr int kC4MaxTokensPerWave = 8;      // 8 tokens x 8 window rows = the 64 lanes
constexpr int kC4TargetWaves = 2048;        // 2 waves per SIMD on 256 CUs
constexpr int kC4WideTargetWaves = 3072;    // 3 per SIMD: one 12-wave workgroup per CU
constexpr int kC4WideMaxGatedPerWave = 64;   // wide waves gate up to 64 tokens (a lane each of the
                                             // workgroup's threads) and stage 16 records a round
constexpr int kC4WavesPerSimd = 3;          // room for all 32 window loads in flight

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

// Load NR window rows (wave-uniform row pointers, already offset to the row's kv half) and
// pool the lane's 8 columns into c[0..3] (v0) and c[4..7] (v1); all 4*NR loads are issued
// before the first use.
template <int NR, int HALVES = 1>
__device__ __forceinline__ void pool_rows(const float* const (&rowp)[NR], uint32_t col,
                                          float (&c)[8]) {
#pragma unroll
  for (int h = 0; h < HALVES; ++h) {
    constexpr int NV = 2 / HALVES;  // column vectors per phase
    float4 kv[NV][NR], sc[NV][NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint32_t off = col + 256u * static_cast<uint32_t>(h * NV + v);
        kv[v][r] = load_stream(rowp[r] + off);
        sc[v][r] = load_stream(rowp[r] + kC4ScoreOffset + off);
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float s[NR], x[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float4& a = sc[v][r];
          const float4& b = kv[v][r];
          s[r] = (k == 0 ? a.x : k == 1 ? a.y : k == 2 ? a.z : a.w) * kLog2e;
          x[r] = k == 0 ? b.x : k == 1 ? b.y : k == 2 ? b.z : b.w;
        }
        c[4 * (h * NV + v) + k] = pool_column<NR>(s, x);
      }
    }
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

// The lane's index in its wave (0..63), counted by mbcnt, which reads no work-item id register.
// Written as a volatile asm statement so that the compiler recounts it where it is used instead
// of hoisting it out of a loop and keeping it live (or spilled) across the loop.
__device__ __forceinline__ int lane_index() {
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  return ln;
}

__device__ __forceinline__ uint8_t scale_byte(int e) {
  const int b = e + 127;
  return static_cast<uint8_t>(b < 0 ? 0 : (b > 255 ? 255 : b));
}

template <bool kDebug, int WPE, int NW, int NB>
__global__ void __launch_bounds__(64 * NW)
    __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
    c4_compress_store_kernel(const C128Params p, int32_t state_bs, int32_t state_bs_log2,
                             int32_t tokens_per_wave) {
  // A wave takes up to 8 * NB tokens a round, resolved in NB batches of 8 (its 64 metadata lanes:
  // 8 tokens x 8 window rows); NB = 2 only for wide workgroups.
  constexpr bool kDeal = NW > kC4NarrowWaves;
  static_assert(NB == 1 || (NB == 2 && kDeal), "two batches only in wide workgroups");
  constexpr int kMaxTok = kC4MaxTokensPerWave * NB;
  __shared__ __align__(16) uint8_t stage_all[NW][kMaxTok * kSlotBytes];
  __shared__ int32_t slot_all[NW][kMaxTok];

  // The token count per wave and the kv-slot pointer sit in another 64-byte line of the kernel
  // arguments than the other pointers; the empty asm makes all of them arrive in one round trip
  // (the compiler otherwise requests that line only after its first wait).
  asm volatile("" ::"s"(tokens_per_wave), "s"(p.kv_slot_mapping), "s"(p.positions),
               "s"(p.rms_w));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* stage = stage_all[wave];
  int32_t* slot_of = slot_all[wave];
  const int64_t tbase = (static_cast<int64_t>(blockIdx.x) * NW + wave) * tokens_per_wave;
  if (lane < kMaxTok) slot_of[lane] = -1;

  // ---- wide workgroups deal their tokens out: one lane per token of the workgroup's range (up
  // to 64 tokens a wave) loads its gate, request id and kv slot; the tokens that pass are listed
  // in LDS and wave w takes list entries w, w + NW, w + 2 NW, ..., so that every wave reads about
  // as many windows before the workgroup's barrier.  A wave's stage holds kMaxTok records, so a
  // wave dealt more tokens than that takes them in rounds, each ending in the workgroup's
  // insert.  Narrow workgroups keep each wave's consecutive tokens, one round.
  constexpr int kDealMax = kDeal ? 64 * NW : 1;
  static_assert(!kDeal || kDealMax <= 64 * NW, "one lane per dealt token");
  __shared__ int32_t deal_tok[kDealMax];
  __shared__ int32_t deal_meta[kDealMax][3];  // position, request, kv slot
  __shared__ int32_t deal_count[NW];
  const int64_t gbase = static_cast<int64_t>(blockIdx.x) * NW * tokens_per_wave;
  int32_t my_tokens = tokens_per_wave;
  int rounds = 1;  // workgroup-uniform
  if constexpr (kDeal) {
    const int tid = static_cast<int>(threadIdx.x);
    bool pass = false;
    int32_t pos = -1, req = -1, kvs = -1;
    if (tid < NW * tokens_per_wave && gbase + tid < p.num_tokens) {
      const int64_t t = gbase + tid;
      pos = p.positions[t];
      const int32_t slot = p.slot_mapping[t];
      req = p.token_to_req[t];
      kvs = p.kv_slot_mapping[t];
      pass = slot >= 0 && pos >= 0 && (pos & (kC4Ratio - 1)) == kC4Ratio - 1;
    }
    const uint64_t passing = __builtin_amdgcn_ballot_w64(pass);
    if (lane == 0) deal_count[wave] = __popcll(passing);
    __syncthreads();
    int before = 0, n = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = deal_count[w];
      before += w < wave ? c : 0;
      n += c;
    }
    if (pass) {
      const int e = before + static_cast<int>(__popcll(passing & ((1ull << lane) - 1)));
      deal_tok[e] = tid;
      deal_meta[e][0] = pos;
      deal_meta[e][1] = req;
      deal_meta[e][2] = kvs;
    }
    __syncthreads();
    my_tokens = n > wave ? (n - wave + NW - 1) / NW : 0;
    // a single-batch wide kernel is launched with at most 8 tokens a wave: one round
    if constexpr (NB > 1) rounds = ((n + NW - 1) / NW + kMaxTok - 1) / kMaxTok;
  }

  // One batch of up to 8 tokens of round `base` (the wave's dealt tokens base + b0 ..), into the
  // wave's stage slots b0 .. b0 + nb - 1.  With two batches
  // the lane index is counted afresh in each, and the state block size is made opaque, so that
  // the loop keeps neither the work-item id, per-lane addresses nor division constants live (and
  // spilled) from one batch to the next.
  const auto batch = [&](const int base, const int b0, const int nb) {
    int ln = lane, sbs = state_bs;
    if constexpr (NB > 1) {
      ln = lane_index();
      asm volatile("" : "+s"(sbs));
    }
    const uint32_t col = static_cast<uint32_t>(ln) * 4;
    const float4 w0 = *reinterpret_cast<const float4*>(p.rms_w + col);
    const float4 w1 = *reinterpret_cast<const float4*>(p.rms_w + 256 + col);
    const int j = ln & 15;  // RoPE pair index of lanes 48..63
    const int mk = ln >> 3, mi = ln & 7;

    // ---- metadata of the batch's tokens, one lane per (token k, window row i): gate, request,
    // block column, block id and their range checks.  The request id and the kv slot come with
    // the gate's position and slot, so the block ids wait for one round trip.  A token goes on
    // only if every one of its 8 lanes passes.  Rows before position 0 (pos 3, i < 4) are not
    // read and need no block.
    int32_t mpos = -1, mkv = -1;
    int64_t moff = 0;
    bool mok = false;
    bool gate = false;
    int32_t req = -1, kvs = -1;
    if constexpr (kDeal) {
      if (mk < nb) {
        const int e = wave + NW * (base + b0 + mk);
        mpos = deal_meta[e][0];
        req = deal_meta[e][1];
        kvs = deal_meta[e][2];
        gate = true;
      }
    } else {
      const int64_t mt = tbase + mk;  // narrow: a single batch, b0 = 0
      if (mk < tokens_per_wave && mt < p.num_tokens) {
        mpos = p.positions[mt];
        const int32_t slot = p.slot_mapping[mt];
        req = p.token_to_req[mt];
        kvs = mi == 0 ? p.kv_slot_mapping[mt] : -1;
        gate = slot >= 0 && mpos >= 0 && (mpos & (kC4Ratio - 1)) == kC4Ratio - 1;
      }
    }
    if (gate) {
      mok = req >= 0 && req < p.bt_rows && mpos / sbs < p.bt_cols &&
            (mpos & ~(kC4Ratio - 1)) < p.cs_rows;
      const int32_t q = mpos - (kC4Rows - 1) + mi;
      if (mok && q >= 0) {
        const int32_t bcol = state_bs_log2 >= 0 ? q >> state_bs_log2 : q / sbs;
        const int32_t boff = q - bcol * sbs;
        const int32_t b = p.block_table[static_cast<int64_t>(req) * p.bt_stride + bcol];
        mok = static_cast<uint32_t>(b) < static_cast<uint32_t>(p.n_state_blocks);
        moff = static_cast<int64_t>(b) * p.s0 + static_cast<int64_t>(boff) * p.s1 +
               (mi >= kC4Ratio ? kHead : 0);
      }
      mkv = kvs;
    }
    const uint64_t good = __builtin_amdgcn_ballot_w64(mok);

    for (int k = 0; k < nb; ++k) {
      if (((good >> (8 * k)) & 0xffu) != 0xffu) continue;  // inactive or an index out of range
      const int slot_k = b0 + k;  // the token's place in the wave's stage
      const int32_t pos = __builtin_amdgcn_readlane(mpos, 8 * k);
      const int32_t kv_slot = __builtin_amdgcn_readlane(mkv, 8 * k);
      const int32_t rope_row = pos & ~(kC4Ratio - 1);  // (pos // 4) * 4
      const float* rowp[kC4Rows];
  #pragma unroll
      for (int i = 0; i < kC4Rows; ++i) {
        const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(moff), 8 * k + i);
        const uint32_t hi =
            __builtin_amdgcn_readlane(static_cast<uint32_t>(static_cast<uint64_t>(moff) >> 32),
                                      8 * k + i);
        rowp[i] = p.state + static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
      }
      const float* cs = p.cos_sin + static_cast<int64_t>(rope_row) * p.cs_stride;
      const float cos0 = cs[2 * j], cos1 = cs[2 * j + 1];
      const float sin0 = cs[kRope / 2 + 2 * j], sin1 = cs[kRope / 2 + 2 * j + 1];

      // ---- pool: 8 rows, or only the current window's 4 at position 3
      float c[8];
      if (pos >= kC4Rows - 1) {
        pool_rows<kC4Rows>(rowp, col, c);
      } else {
        const float* const cur[kC4Ratio] = {rowp[4], rowp[5], rowp[6], rowp[7]};
        pool_rows<kC4Ratio>(cur, col, c);
      }

      // ---- RMSNorm over the 512 columns (one wave)
      float ss = 0.0f;
  #pragma unroll
      for (int m = 0; m < 8; ++m) ss = __builtin_fmaf(c[m], c[m], ss);
      ss = wave_sum(ss);
      const float rrms = 1.0f / __builtin_sqrtf(ss * (1.0f / kHead) + p.eps);
      const float n[8] = {c[0] * rrms * w0.x, c[1] * rrms * w0.y, c[2] * rrms * w0.z,
                          c[3] * rrms * w0.w, c[4] * rrms * w1.x, c[5] * rrms * w1.y,
                          c[6] * rrms * w1.z, c[7] * rrms * w1.w};
      if constexpr (kDebug) {
        const int64_t t = kDeal ? gbase + deal_tok[wave + NW * (base + slot_k)] : tbase + k;
        float* out = p.compressed_out + t * kHead;
        *reinterpret_cast<float4*>(out + col) = make_float4(c[0], c[1], c[2], c[3]);
        *reinterpret_cast<float4*>(out + 256 + col) = make_float4(c[4], c[5], c[6], c[7]);
      }
      if (kv_slot < 0 || kv_slot >= p.n_kv_slots) continue;

      // ---- per-64 absmax of the bf16-rounded values, UE8M0 / E4M3, RoPE -> this token's
      // 584-byte slot in the wave's LDS stage
      float u[8];
  #pragma unroll
      for (int m = 0; m < 8; ++m) u[m] = bf16_round(n[m]);
      const float a0 = group16_max(__builtin_fmaxf(
          __builtin_fmaxf(__builtin_fabsf(u[0]), __builtin_fabsf(u[1])),
          __builtin_fmaxf(__builtin_fabsf(u[2]), __builtin_fabsf(u[3]))));
      const float a1 = group16_max(__builtin_fmaxf(
          __builtin_fmaxf(__builtin_fabsf(u[4]), __builtin_fabsf(u[5])),
          __builtin_fmaxf(__builtin_fabsf(u[6]), __builtin_fabsf(u[7]))));
      uint8_t* rec = stage + slot_k * kSlotBytes;
      uint8_t* scl = rec + kRecordBytes;
      const int group = ln >> 4;
      // v0: columns 0..255, quant blocks 0..3
      const int e0 = ue8m0_exponent(a0);
      *reinterpret_cast<uint32_t*>(rec + col) = quant4(u, 0, e0);
      if ((ln & 15) == 0) scl[group] = scale_byte(e0);
      if (ln < 48) {
        // v1: columns 256..447, quant blocks 4..6
        const int e1 = ue8m0_exponent(a1);
        *reinterpret_cast<uint32_t*>(rec + 256 + col) = quant4(u, 4, e1);
        if ((ln & 15) == 0) scl[4 + group] = scale_byte(e1);
      } else {
        // v1 of lanes 48..63: RoPE dims 448 + 4j .. +3, pairs 2j and 2j + 1
        const float x0 = n[4] * cos0 - n[5] * sin0;
        const float y0 = n[5] * cos0 + n[4] * sin0;
        const float x1 = n[6] * cos1 - n[7] * sin1;
        const float y1 = n[7] * cos1 + n[6] * sin1;
        const uint32_t lo = bf16_bits(x0) | (bf16_bits(y0) << 16);
        const uint32_t hi = bf16_bits(x1) | (bf16_bits(y1) << 16);
        *reinterpret_cast<uint2*>(rec + kNope + 8 * j) = make_uint2(lo, hi);
        if (j == 0) scl[kNumQuant] = 0;  // pad byte
      }
      if (ln == 0) slot_of[slot_k] = kv_slot;
    }
  };
  for (int r = 0; r < (NB > 1 ? rounds : 1); ++r) {
    const int base = r * kMaxTok;
    const int left = my_tokens - base;
    const int mine = left < 0 ? 0 : (left < kMaxTok ? left : kMaxTok);
    if constexpr (NB > 1) {
      for (int b0 = 0; b0 < mine; b0 += 8) batch(base, b0, mine - b0 < 8 ? mine - b0 : 8);
    } else {
      batch(base, 0, mine);
    }

    // ---- paged insert of every staged record, after the last state read of every wave of the
    // workgroup: the k_cache writes reach HBM in bursts instead of interleaved with the read
    // stream (8-byte stores; records and scale groups are 8-byte aligned).  A wave's stage and
    // slot list are its own, so the next round may refill them without a further barrier.
    __syncthreads();
    const int fl = NB > 1 ? lane_index() : lane;
    for (int k = 0; k < (kDeal ? kMaxTok : tokens_per_wave); ++k) {
      const int32_t kv_slot = slot_of[k];
      if (kv_slot < 0) continue;
      const int32_t kb = kv_slot / p.kv_bs;
      const int32_t ko = kv_slot - kb * p.kv_bs;
      uint8_t* blockp = p.k_cache + static_cast<int64_t>(kb) * p.kc_stride0;
      uint8_t* grec = blockp + static_cast<int64_t>(ko) * kRecordBytes;
      uint8_t* gscl = blockp + static_cast<int64_t>(p.kv_bs) * kRecordBytes +
                      static_cast<int64_t>(ko) * kScaleBytes;
      const uint8_t* rec = stage + k * kSlotBytes;
      *reinterpret_cast<uint2*>(grec + 8 * fl) = *reinterpret_cast<const uint2*>(rec + 8 * fl);
      if (fl < 8)
        *reinterpret_cast<uint2*>(grec + 512 + 8 * fl) =
            *reinterpret_cast<const uint2*>(rec + 512 + 8 * fl);
      else if (fl == 8)
        *reinterpret_cast<uint2*>(gscl) = *reinterpret_cast<const uint2*>(rec + kRecordBytes);
    }
    if (r + 1 < rounds && fl < kMaxTok) slot_of[fl] = -1;
  }
}

// Tokens per wave: enough waves for the target (2 per SIMD for the narrow shape, 3 for the wide
// one) before a wave takes more than one token; at most max_tokens (8 for a narrow wave, the
// 64 lanes of its metadata; 64 for a wide wave, which gates one token a thread).
int c4_tokens_per_wave(int64_t num_tokens, int64_t target_waves, int64_t max_tokens) {
  const int64_t k = (num_tokens + target_waves - 1) / target_waves;
  return static_cast<int>(k < 1 ? 1 : (k > max_tokens ? max_tokens : k));
}

template <int NW, int NB>
hipError_t launch_c4_as(const C128Params& p, int32_t state_bs, int32_t kpw, hipStream_t stream) {
  const int64_t waves = (static_cast<int64_t>(p.num_tokens) + kpw - 1) / kpw;
  const dim3 grid(static_cast<unsigned>((waves + NW - 1) / NW));
  const dim3 block(64 * NW);
  const int32_t lg = (state_bs & (state_bs - 1)) == 0 ? __builtin_ctz(state_bs) : -1;
  if (p.compressed_out)
    return launch_kernel(c4_compress_store_kernel<true, kC4WavesPerSimd, NW, NB>, grid, block,
                         stream, p, state_bs, lg, kpw);
  return launch_kernel(c4_compress_store_kernel<false, kC4WavesPerSimd, NW, NB>, grid, block,
                       stream, p, state_bs, lg, kpw);
}

}  // namespace

// Small batches take 4-wave workgroups, spread over as many CUs as possible.  From
// kC4WideMinTokens on, while one round of them covers the batch, a workgroup is 12 waves (one
// per CU), so that the records of a whole CU wait in LDS until all of its waves have read their
// windows: the record writes then meet far less of the read stream.  A wide wave gates up to 64
// tokens (cu_count * 768 tokens in one round of workgroups) and stages 16 records at a time: a
// chunked prefill, where about one token in four writes, stays at one insert per workgroup up to
// about 200k tokens, and a denser batch beyond 49,152 tokens inserts after every 16 records a
// wave.  Beyond one round the narrow shape stays, as a second round of wide workgroups would run
// as a tail.
hipError_t launch_c4_compress_store(const C128Params& p, int32_t state_bs, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  if (p.num_tokens >= kC4WideMinTokens) {
    const int32_t kpw =
        c4_tokens_per_wave(p.num_tokens, kC4WideTargetWaves, kC4WideMaxGatedPerWave);
    const int64_t waves = (static_cast<int64_t>(p.num_tokens) + kpw - 1) / kpw;
    if ((waves + kC4WideWaves - 1) / kC4WideWaves <= device_cu_count()) {
      // one batch of metadata per wave while 8 tokens a wave suffice: the single-batch kernel
      // keeps half the LDS stage and fewer registers
      if (kpw <= kC4MaxTokensPerWave)
        return launch_c4_as<kC4WideWaves, 1>(p, state_bs, kpw, stream);
      return launch_c4_as<kC4WideWaves, 2>(p, state_bs, kpw, stream);
    }
  }
  return launch_c4_as<kC4NarrowWaves, 1>(
      p, state_bs, c4_tokens_per_wave(p.num_tokens, kC4TargetWaves, kC4MaxTokensPerWave), stream);
}

}  // namespace dsv4
