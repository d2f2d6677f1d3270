// Other schedules of the C128 compress-store for MI355X (gfx950): the same per-token
// computation as the single pass in c128_kernel.hip (gate, window gather, per-column softmax
// pooling, RMSNorm, UE8M0/E4M3 quantisation, GPT-J RoPE, paged insert; vLLM
// "fused_compress_quant_cache" API page, sparse-attention fused kernel), distributed
// differently over workgroups:
//
//  * fan-out, for decode batches of up to about a hundred tokens, where one workgroup per token
//    leaves most CUs idle: a token's window is split over several workgroups, and the last of
//    them to finish merges their partial softmax states;
//  * compacted, for long varlen (prefill) batches where about one token in 128 closes a window:
//    a gate scan lists those tokens, and a persistent grid processes only them;
//  * staged, which the plain entry point takes from 2048 tokens on: a workgroup takes up to 64
//    tokens and inserts their records after its last state read, so that the k_cache writes do
//    not land in the middle of the state stream.

#include <atomic>
#include <mutex>

#include "c128_device.h"
#include "c128_launch.h"

// Scratch of the allocation-free compacted schedule (launch_c128_compacted_static): the scan
// blocks' counts, then the compacted token list, for at most kStaticCompactedMaxTokens tokens
// (4 MiB + 4 KiB).  Each device holds its own copy for the life of the process.  Host code must
// not pass this name to a kernel (on the host it is only a stand-in for the symbol): it takes
// the device address from hipGetSymbolAddress, once per device.
static __device__ __align__(256) int32_t
    scratch[dsv4::kStaticCompactedScanBlocks + dsv4::kStaticCompactedMaxTokens];

namespace dsv4 {
namespace {

// ---------------------------------------------------------------------------------------------
// Pieces of the fan-out and compacted kernels.  The single-pass kernel (c128_kernel.hip) keeps
// its own inline form of the same steps, which the compiler schedules better for the
// large-batch stream.

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
  // The request id is loaded with the gate's loads (one dependent round trip less before the
  // block ids), and its sign test joins the gate's tests in one branch: with the gate
  // branching first, the compiler sinks the request load below it, into a round trip of its own.
  const int32_t req = p.token_to_req[t];
  if ((slot < 0) | (pos < 0) | ((pos & (kRatio - 1)) != kRatio - 1) | (req < 0)) return w;
  const int32_t win = pos >> 7;  // window rows 128*win .. 128*win + 127
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

// LDS copies of the epilogue's inputs besides the pooled state: the two column halves of rms_w,
// the token's cos/sin row and, for each epilogue wave, the kv slot.
struct EpilogueInputs {
  float4 w[2][64];
  float cs[kRope];
  int32_t kv[2];
};

// Fetch them with loads that write LDS directly: every lane of both epilogue waves (column
// half `half`).  A kernel issues this early, where the round trip overlaps other waiting, and
// waits for the loads (vmcnt) before any of its waves can exit.  The compiler treats these
// loads as writes to any memory, so the kernel issues them after its last block-id read.
__device__ __forceinline__ void fetch_epilogue_inputs(const C128Params& p, int32_t t,
                                                      int32_t rope_row, int half, int lane,
                                                      EpilogueInputs& e) {
  load_to_lds16(p.rms_w + half * 256 + lane * 4, &e.w[half][0]);
  if (half == 1)
    load_to_lds4(p.cos_sin + static_cast<int64_t>(rope_row) * p.cs_stride + lane, e.cs);
  if (lane == 0) load_to_lds4(p.kv_slot_mapping + t, &e.kv[half]);
}

// Fused epilogue of token t on 128 lanes (2 waves, one per column half; 4 columns per lane):
// RMSNorm, bf16 round trip, per-64 absmax -> UE8M0 exponent -> E4M3FN codes, GPT-J RoPE ->
// bf16, paged insert.  sumsq is the sum of squares of all 512 pooled values.  The 584-byte
// record goes to the token's k_cache slot, or with kStage to `stage` (an LDS record: 576 data
// bytes, then the 8 scale bytes) for a later insert.  Returns the kv slot, or -1 when the token
// has none (nothing is written then).  With `in`, rms_w, the kv slot and the cos/sin row come
// from its LDS copies (fetch_epilogue_inputs) instead of global memory.
template <bool kDebug, bool kStage = false>
__device__ __forceinline__ int32_t epilogue(const C128Params& p, int32_t t, int32_t rope_row,
                                            const float (&c)[4], int half, int lane, int col,
                                            float sumsq, uint8_t* stage = nullptr,
                                            const EpilogueInputs* in = nullptr) {
  const float var = sumsq * (1.0f / kHead);
  const float rrms = 1.0f / __builtin_sqrtf(var + p.eps);
  const float4 w = in ? in->w[half][lane] : *reinterpret_cast<const float4*>(p.rms_w + col);
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

  const int32_t kv_slot = in ? in->kv[half] : p.kv_slot_mapping[t];
  if (kv_slot < 0 || kv_slot >= p.n_kv_slots) return -1;
  uint8_t* rec;
  uint8_t* scl;
  if constexpr (kStage) {
    rec = stage;
    scl = stage + kRecordBytes;
  } else {
    const int32_t kb = kv_slot / p.kv_bs;
    const int32_t ko = kv_slot - kb * p.kv_bs;
    uint8_t* blockp = p.k_cache + static_cast<int64_t>(kb) * p.kc_stride0;
    rec = blockp + static_cast<int64_t>(ko) * kRecordBytes;
    scl = blockp + static_cast<int64_t>(p.kv_bs) * kRecordBytes +
          static_cast<int64_t>(ko) * kScaleBytes;
  }

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
    const float* cs = in ? in->cs : p.cos_sin + static_cast<int64_t>(rope_row) * p.cs_stride;
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
  return kv_slot;
}

// c = acc / l, then the RMSNorm sum of squares over both column halves (one barrier), then the
// epilogue on the 128 lanes of the first two waves.  Every wave must call it.  Returns the
// epilogue's kv slot on the epilogue waves, -1 on the others.
template <bool kDebug, bool kStage = false>
__device__ __forceinline__ int32_t finish_token(const C128Params& p, int32_t t, int32_t rope_row,
                                                bool epilogue_wave, int half, int lane, int col,
                                                const float (&l)[4], const float (&acc)[4],
                                                float* lds_ss, uint8_t* stage = nullptr,
                                                const EpilogueInputs* in = nullptr) {
  float c[4] = {0.f, 0.f, 0.f, 0.f};
  if (epilogue_wave) {
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = acc[k] / l[k];
    float ss = c[0] * c[0] + c[1] * c[1] + c[2] * c[2] + c[3] * c[3];
    ss = wave_sum(ss);
    if (lane == 0) lds_ss[half] = ss;
  }
  __syncthreads();
  if (!epilogue_wave) return -1;
  return epilogue<kDebug, kStage>(p, t, rope_row, c, half, lane, col, lds_ss[0] + lds_ss[1],
                                  stage, in);
}

// 16 bytes as two 8-byte agent-scope atomic accesses (relaxed): coherent across the XCDs
// within a kernel.  p is 8-byte aligned.
__device__ __forceinline__ void store_agent4(float* p, float a, float b, float c, float d) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  const uint64_t lo = static_cast<uint64_t>(__float_as_uint(a)) |
                      (static_cast<uint64_t>(__float_as_uint(b)) << 32);
  const uint64_t hi = static_cast<uint64_t>(__float_as_uint(c)) |
                      (static_cast<uint64_t>(__float_as_uint(d)) << 32);
  __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float4 load_agent4(const float* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float4(__uint_as_float(static_cast<uint32_t>(lo)),
                     __uint_as_float(static_cast<uint32_t>(lo >> 32)),
                     __uint_as_float(static_cast<uint32_t>(hi)),
                     __uint_as_float(static_cast<uint32_t>(hi >> 32)));
}

// ---------------------------------------------------------------------------------------------
// Fan-out for small batches, one kernel: a token's 16 window blocks are split over
// S = 16 / (RG*NBW) workgroups (grid = T x S).  Workgroup (t, s) streams window blocks
// s*RG*NBW .. (s+1)*RG*NBW - 1 (NBW blocks for each of its RG row groups), merges its row groups
// and writes its partial state to the workspace:
//   partials[((t * S + s) * 3 + {0: m (log2 units), 1: l, 2: acc}) * 512 + column],
// then adds 1 to the token's arrival counter.  The workgroup that brings the counter to S is the
// last of the token: it folds the S partials in split order, runs the epilogue and puts the
// counter back to 0, so every call leaves the counters as it found them.
//
// Cross-workgroup visibility without cache-wide fences.  The 8 XCDs' L2 caches are not coherent
// with each other inside a kernel, and an agent-scope release/acquire fence pair would write
// back and invalidate a whole L2 per workgroup (which serialises hundreds of workgroups).
// Instead the partial states are written with agent-scope atomic stores and read with
// agent-scope atomic loads (device-coherent accesses that do not rely on the L2 line state), and
// each wave waits for its stores to complete (s_waitcnt) before the workgroup barrier that
// precedes the counter update; the last workgroup only reads partials after its own counter
// update returned S - 1.  No workgroup ever waits for another, so the kernel cannot stall.
template <int RG, int NBW, int CH, bool kDebug>
__global__ void __launch_bounds__(128 * RG) c128_fanout_kernel(const C128Params p,
                                                             float* __restrict__ partials,
                                                             uint32_t* __restrict__ counters) {
  constexpr int kBlocksPerGroup = RG * NBW;
  static_assert(kWindowBlocks % kBlocksPerGroup == 0, "splits must divide the window");
  constexpr int S = kWindowBlocks / kBlocksPerGroup;

  __shared__ float4 lds_ml[RG][2][64];
  __shared__ float4 lds_l[RG][2][64];
  __shared__ float4 lds_acc[RG][2][64];
  __shared__ float lds_ss[2];
  __shared__ uint32_t lds_last;
  __shared__ EpilogueInputs lds_in;

  const int32_t t = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave & 1;
  const int rg = wave >> 1;
  const int col = half * 256 + lane * 4;

  // Every workgroup of a token takes the same decision here, so either all S of them reach the
  // counter or none does.
  const Window win = gate_and_window(p, t);
  if (!win.ok) return;

  float ml[4], l[4], acc[4];
  stream_blocks<NBW, CH>(p, win.bt + s * kBlocksPerGroup + rg * NBW, static_cast<uint32_t>(col),
                         ml, l, acc);
  merge_row_groups<RG>(lds_ml, lds_l, lds_acc, rg, half, lane, ml, l, acc);

  // Any workgroup of the token may turn out to be the last, so each fetches the epilogue's
  // inputs; their round trip overlaps the handoff's, and the wait below covers them.
  float* base = partials + static_cast<int64_t>(t) * S * (3 * kHead) + col;
  if (rg == 0) {
    fetch_epilogue_inputs(p, t, win.rope_row, half, lane, lds_in);
    float* out = base + s * (3 * kHead);
    store_agent4(out, ml[0], ml[1], ml[2], ml[3]);
    store_agent4(out + kHead, l[0], l[1], l[2], l[3]);
    store_agent4(out + 2 * kHead, acc[0], acc[1], acc[2], acc[3]);
  }
  // This wave's partial stores have completed before the barrier.  An asm statement with a
  // memory clobber, so the compiler cannot move the stores below it (the s_waitcnt builtin
  // does not constrain memory operations).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t arrived =
        __hip_atomic_fetch_add(counters + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    const uint32_t last = arrived == static_cast<uint32_t>(S);
    if (last) __hip_atomic_store(counters + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_last = last;
  }
  __syncthreads();
  if (!lds_last) return;

  if (rg == 0) {
    const float4 m0 = load_agent4(base);
    const float4 l0 = load_agent4(base + kHead);
    const float4 a0 = load_agent4(base + 2 * kHead);
    ml[0] = m0.x; ml[1] = m0.y; ml[2] = m0.z; ml[3] = m0.w;
    l[0] = l0.x; l[1] = l0.y; l[2] = l0.z; l[3] = l0.w;
    acc[0] = a0.x; acc[1] = a0.y; acc[2] = a0.z; acc[3] = a0.w;
#pragma unroll
    for (int q = 1; q < S; ++q) {
      const float* in = base + q * (3 * kHead);
      fold(ml, l, acc, load_agent4(in), load_agent4(in + kHead), load_agent4(in + 2 * kHead));
    }
  }
  finish_token<kDebug>(p, t, win.rope_row, rg == 0, half, lane, col, l, acc, lds_ss, nullptr,
                       &lds_in);
}

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


// ---------------------------------------------------------------------------------------------
// Staged schedule (the plain entry point from 2048 tokens on).  With one workgroup per token,
// each token's 584-byte record reaches HBM on its own, in the middle of the state stream; on
// MI355X those scattered writes cost about 4.5% of the large-batch call (measured: the single
// pass with its stores switched off runs at the rate of a pure read of the same gather).  Here a
// workgroup of 8 row groups (16 waves, one window block per wave at a time) streams a share of
// the active tokens, keeps their records in LDS and inserts them after the last state read of
// each stage of up to KMAX tokens, so the k_cache writes leave the state stream.
//
//  * One round: the grid is one workgroup per CU (the LDS stage allows no second one), so no
//    workgroup ever waits for a CU to free up.
//  * Balanced by rank.  Every workgroup tests the gate of every token (position and state slot:
//    8 bytes a token, served from L2 once the first workgroups have fetched them) and counts the
//    tokens that pass per count block of `block_tokens` consecutive tokens, in LDS; the
//    exclusive prefix of those counts gives each passing token its rank, its index in token
//    order among the passing tokens, the same in every workgroup.  Workgroup b of G takes ranks
//    [A*b/G, A*(b+1)/G) of the A passing tokens: every workgroup streams the same number of
//    windows, within one, whether every token closes a window (a decode batch: 64 consecutive
//    tokens each at 16384) or one in 128 does (chunked prefill: one or two each).
//  * A stage takes up to KMAX of the workgroup's ranks.  Its tokens are located by reading the
//    gates of only the count blocks that hold those ranks again.  Then one thread per (token,
//    window block) resolves request, window column, RoPE row and block id into LDS, and wave 0
//    lists the tokens whose indices are all in range.  Inside the token loop every per-token
//    value comes from LDS: a global load after a workgroup barrier cannot be a scalar load (the
//    barrier's fence counts as a possible write), and a chain of vector loads with full waits in
//    front of every token costs more than the staging gains.
//  * Per token, the same steps as the single pass (stream, row-group merge, fused epilogue);
//    8 row groups instead of 4, so the fp32 summation order differs from the single pass's.
constexpr int kStagedCountBlocks = 4096;  // most count blocks (LDS: one int32 each)
constexpr int kCountUnroll = 12;          // 256-token chunks a wave gates at once
constexpr int kMaskChunks = 1280;         // batches of up to this many chunks keep gate masks
constexpr int kLocateUnroll = 4;

__device__ __forceinline__ bool gate_of(int32_t pos, int32_t slot) {
  return (slot >= 0) & (pos >= 0) & ((pos & (kRatio - 1)) == kRatio - 1);
}

__device__ __forceinline__ bool gate_open(const C128Params& p, int32_t t) {
  return gate_of(p.positions[t], p.slot_mapping[t]);
}

// Gates of U sub-tiles of 64 tokens, sub-tile u starting at token first + u * stride (lane l:
// token + l).  Every load is issued before any result is used: indices past the batch are
// clamped to its last token and their gate is closed afterwards.
template <int U>
__device__ __forceinline__ void gate_tiles(const C128Params& p, int32_t T, int32_t first,
                                           int32_t stride, int32_t end, int lane,
                                           bool (&act)[U]) {
  int32_t pos[U], slot[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t t = first + u * stride + lane;
    const int32_t tc = t < T ? t : T - 1;
    pos[u] = p.positions[tc];
    slot[u] = p.slot_mapping[tc];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) act[u] = (first + u * stride + lane < end) & gate_of(pos[u], slot[u]);
}

// The work-item id passed through an empty asm statement.  Per-thread addresses computed from it
// inside a loop are recomputed there (a few VALU instructions) instead of being hoisted out and
// kept live, or spilled to scratch, across the window stream.
__device__ __forceinline__ int fresh_tid() {
  int t = static_cast<int>(__builtin_amdgcn_workitem_id_x());
  asm volatile("" : "+v"(t));
  return t;
}

// The last count block whose first rank is <= r, the block that holds rank r (r < A), by one
// wave in two ballot steps over the non-decreasing prefix: lane l first tests block l * step
// (step = ceil(nblocks / 64) <= 64), then block c1 + l within the step that holds the answer.
__device__ __forceinline__ int block_of_rank(const int32_t* pre, int nblocks, int32_t r,
                                             int lane) {
  const int step = (nblocks + 63) >> 6;
  const int c = lane * step;
  const uint64_t m1 = __builtin_amdgcn_ballot_w64(c < nblocks && pre[c < nblocks ? c : 0] <= r);
  const int c1 = (63 - __builtin_clzll(m1)) * step;  // pre[0] = 0 <= r: m1 has bit 0
  const int c2 = c1 + lane;
  const uint64_t m2 = __builtin_amdgcn_ballot_w64(lane < step && c2 < nblocks &&
                                                  pre[c2 < nblocks ? c2 : 0] <= r);
  return c1 + (63 - __builtin_clzll(m2));              // lane 0 (block c1) always passes
}

template <int RG, int CH, int WPE, int KMAX, bool kDebug>
__global__ void __launch_bounds__(128 * RG) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
c128_staged_kernel(const C128Params p, int32_t block_tokens, int32_t nblocks) {
  static_assert(kWindowBlocks % RG == 0, "row groups must split the 16 window blocks");
  static_assert(kStateBlock % CH == 0, "a stage must not straddle two state blocks");
  static_assert(KMAX * kWindowBlocks <= 128 * RG, "one resolve thread per (token, block)");
  static_assert(KMAX <= 64, "wave 0 lists a stage's tokens, one lane each");
  static_assert(kStagedCountBlocks <= 4 * 128 * RG, "the prefix takes four counts a thread");
  constexpr int NW = 2 * RG;    // waves
  constexpr int NT = 64 * NW;   // threads
  constexpr int NB = kWindowBlocks / RG;  // state blocks per wave
  constexpr int NCH = NB * kStateBlock / CH;
  constexpr int kStagesPerBlock = kStateBlock / CH;
  static_assert(NCH % 2 == 0, "ping-pong needs an even chunk count");

  __shared__ float4 lds_ml[RG][2][64];
  __shared__ float4 lds_l[RG][2][64];
  __shared__ float4 lds_acc[RG][2][64];
  __shared__ float lds_ss[2];
  __shared__ int32_t lds_pre[kStagedCountBlocks];  // per count block: passing tokens, then the
                                                   // rank of its first passing token
  __shared__ int32_t lds_wsum[NW];
  __shared__ uint64_t lds_mask[kMaskChunks][4];  // per 256-token chunk: ballot j holds the gate of
                                                 // token 4l + j in bit l
  __shared__ __align__(16) int32_t lds_ids[KMAX][kWindowBlocks];  // -1: out of range
  __shared__ int32_t lds_tok[KMAX];   // the stage's tokens, in rank order
  __shared__ int32_t lds_rope[KMAX];  // RoPE row; -1: the token is skipped
  __shared__ int32_t lds_kv[KMAX];    // kv slot of a staged record; -1: none
  __shared__ int32_t lds_list[KMAX];  // 1: the stage entry has every index in range
  __shared__ __align__(16) uint8_t lds_stage[KMAX][kSlotBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave & 1;
  const int rg = wave >> 1;
  const int32_t T = p.num_tokens;  // at most 2^27: tokens and ranks fit in 32 bits

  // ---- count pass: tokens that pass the gate, per count block.  The batch is read in chunks of
  // 256 tokens: lane l gates tokens 4l .. 4l + 3 of a chunk with one 16-byte load of positions
  // and one of state slots (per-lane 4-byte loads cost the address unit as much per instruction
  // for a quarter of the bytes, which made the pass 4x slower).  Wave w takes the full chunks
  // w, w + NW, ..., kCountUnroll of them at a time, every load issued before any gate is
  // evaluated; each workgroup starts its walk at its own chunk, spread over the batch.  Wave 0
  // then gates the last, partial chunk; arrays that are not 16-byte aligned take 4-byte loads.
  // Up to kMaskChunks chunks (count blocks of one chunk each), the pass keeps every chunk's gate
  // masks in LDS and the stages rank their tokens from them; beyond, it adds counts per block
  // and the stages read the gates of their blocks again.
  const int32_t nchunk = (T + 255) >> 8;
  const int32_t nfull = T >> 8;
  const bool masked = nchunk <= kMaskChunks && block_tokens == 256;
  const int32_t chunk_per_block = block_tokens >> 8;
  if (!masked)
    for (int c = threadIdx.x; c < nblocks; c += NT) lds_pre[c] = 0;
  __syncthreads();
  auto record = [&](int32_t chunk, bool g0, bool g1, bool g2, bool g3) {
    const uint64_t m0 = __builtin_amdgcn_ballot_w64(g0);
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(g1);
    const uint64_t m2 = __builtin_amdgcn_ballot_w64(g2);
    const uint64_t m3 = __builtin_amdgcn_ballot_w64(g3);
    if (masked) {
      if (lane < 4) lds_mask[chunk][lane] = lane == 0 ? m0 : lane == 1 ? m1 : lane == 2 ? m2 : m3;
    } else {
      const int n = __builtin_popcountll(m0) + __builtin_popcountll(m1) +
                    __builtin_popcountll(m2) + __builtin_popcountll(m3);
      if (n != 0 && lane == 0) atomicAdd(&lds_pre[chunk / chunk_per_block], n);
    }
  };
  // 4-byte gates of the tokens of one chunk that exist
  auto scalar_chunk = [&](int32_t chunk) {
    bool g[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int32_t t = chunk * 256 + 4 * lane + j;
      g[j] = t < T && gate_open(p, t);
    }
    record(chunk, g[0], g[1], g[2], g[3]);
  };
  if (((reinterpret_cast<uintptr_t>(p.positions) |
        reinterpret_cast<uintptr_t>(p.slot_mapping)) & 15) == 0) {
    const int32_t start =
        static_cast<int32_t>(static_cast<int64_t>(nfull) * blockIdx.x / gridDim.x);
    const int32_t mine = (nfull - wave + NW - 1) / NW;  // full chunks wave + NW*k
    for (int32_t k0 = 0; k0 < mine; k0 += kCountUnroll) {
      int32_t chunk[kCountUnroll];
      int4 pos[kCountUnroll], slot[kCountUnroll];
#pragma unroll
      for (int u = 0; u < kCountUnroll; ++u) {
        const int32_t cv = wave + NW * (k0 + u) + start;
        chunk[u] = cv >= nfull ? cv - nfull : cv;
        if (k0 + u < mine) {  // wave-uniform
          const int32_t t0 = chunk[u] * 256 + 4 * lane;
          pos[u] = *reinterpret_cast<const int4*>(p.positions + t0);
          slot[u] = *reinterpret_cast<const int4*>(p.slot_mapping + t0);
        }
      }
#pragma unroll
      for (int u = 0; u < kCountUnroll; ++u)
        if (k0 + u < mine)
          record(chunk[u], gate_of(pos[u].x, slot[u].x), gate_of(pos[u].y, slot[u].y),
                 gate_of(pos[u].z, slot[u].z), gate_of(pos[u].w, slot[u].w));
    }
    if (wave == 0 && nfull < nchunk) scalar_chunk(nfull);
  } else {
    for (int32_t c = wave; c < nchunk; c += NW) scalar_chunk(c);
  }
  __syncthreads();
  // ---- exclusive prefix of the counts (with masks: of the chunks' popcounts): thread i owns
  // blocks 4i .. 4i + 3
  int32_t A;
  {
    int32_t v[4];
    int32_t own = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = threadIdx.x * 4 + k;
      v[k] = c >= nblocks ? 0
             : masked     ? __builtin_popcountll(lds_mask[c][0]) +
                                __builtin_popcountll(lds_mask[c][1]) +
                                __builtin_popcountll(lds_mask[c][2]) +
                                __builtin_popcountll(lds_mask[c][3])
                          : lds_pre[c];
      own += v[k];
    }
    int32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) lds_wsum[wave] = incl;
    __syncthreads();
    int32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int32_t x = lds_wsum[w];
      if (w < wave) before += x;
      total += x;
    }
    int32_t run = before + incl - own;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = threadIdx.x * 4 + k;
      if (c < nblocks) lds_pre[c] = run;
      run += v[k];
    }
    A = __builtin_amdgcn_readfirstlane(total);
    if (threadIdx.x < KMAX) lds_tok[threadIdx.x] = -1;  // entries the locate pass does not fill
  }
  __syncthreads();

  const int64_t G = gridDim.x;
  const int32_t lo = static_cast<int32_t>(static_cast<int64_t>(A) * blockIdx.x / G);
  const int32_t hi = static_cast<int32_t>(static_cast<int64_t>(A) * (blockIdx.x + 1) / G);
  const int col = half * 256 + lane * 4;
  const uint32_t ucol = static_cast<uint32_t>(col);
  const int64_t s0 = p.s0, s1 = p.s1;

  for (int32_t r0 = lo; r0 < hi; r0 += KMAX) {
    const int32_t r1 = r0 + KMAX < hi ? r0 + KMAX : hi;
    const int n = r1 - r0;
    const int tid = fresh_tid();
    const int slane = tid & 63;
    // ---- locate the stage's tokens: the waves share the count blocks that hold ranks
    // r0 .. r1 - 1 and gate their tokens again, in token order
    {
      const int cA = __builtin_amdgcn_readfirstlane(block_of_rank(lds_pre, nblocks, r0, slane));
      const int cB =
          __builtin_amdgcn_readfirstlane(block_of_rank(lds_pre, nblocks, r1 - 1, slane));
      for (int c = cA + wave; c <= cB; c += NW) {
        int32_t run = __builtin_amdgcn_readfirstlane(lds_pre[c]);
        if (masked) {
          // lane l holds tokens 4l .. 4l + 3 of the chunk; their ranks follow the passing tokens
          // of the lanes below, then its own earlier ones
          const uint64_t below = (uint64_t(1) << slane) - 1;
          uint64_t m[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) m[j] = lds_mask[c][j];
          int32_t rank = run;
#pragma unroll
          for (int j = 0; j < 4; ++j) rank += __builtin_popcountll(m[j] & below);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if ((m[j] >> slane) & 1) {
              if (rank >= r0 && rank < r1) lds_tok[rank - r0] = c * 256 + 4 * slane + j;
              ++rank;
            }
          }
          continue;
        }
        const int32_t b0 = c * block_tokens;
        const int32_t b1 = b0 + block_tokens < T ? b0 + block_tokens : T;
        for (int32_t base = b0; base < b1 && run < r1; base += 64 * kLocateUnroll) {
          bool act[kLocateUnroll];
          gate_tiles<kLocateUnroll>(p, T, base, 64, b1, slane, act);
#pragma unroll
          for (int u = 0; u < kLocateUnroll; ++u) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(act[u]);
            const int32_t rank = run + static_cast<int32_t>(__builtin_amdgcn_mbcnt_hi(
                                           static_cast<uint32_t>(m >> 32),
                                           __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m),
                                                                     0u)));
            if (act[u] && rank >= r0 && rank < r1) lds_tok[rank - r0] = base + 64 * u + slane;
            run += __builtin_popcountll(m);
          }
        }
      }
    }
    __syncthreads();
    // ---- resolve: thread (k, i) takes window block i of the stage's k-th token.  The 16
    // threads of a token are 16 consecutive lanes of one wave, so whether all its indices are in
    // range is a 16-lane ballot, with no further barrier.
    {
      const int k = tid / kWindowBlocks, i = tid % kWindowBlocks;
      bool ok = false;
      if (k < n) {
        int32_t rope = -1, id = -1;
        const int32_t t = lds_tok[k];
        const int32_t tc = t >= 0 && t < T ? t : 0;  // position, slot and request in one round trip
        const int32_t pos = p.positions[tc], slot = p.slot_mapping[tc];
        const int32_t req = p.token_to_req[tc];
        if (t >= 0 && t < T && gate_of(pos, slot)) {
          const int32_t win = pos >> 7;  // window rows 128*win .. 128*win + 127
          if (req >= 0 && req < p.bt_rows &&
              static_cast<int64_t>(win + 1) * kWindowBlocks <= p.bt_cols &&
              win * kRatio < p.cs_rows) {
            rope = win * kRatio;
            const int32_t b = p.block_table[static_cast<int64_t>(req) * p.bt_stride +
                                            static_cast<int64_t>(win) * kWindowBlocks + i];
            id = static_cast<uint32_t>(b) < static_cast<uint32_t>(p.n_state_blocks) ? b : -1;
          }
        }
        lds_ids[k][i] = id;
        ok = id >= 0 && rope >= 0;
        if (i == 0) {
          lds_rope[k] = rope;
          lds_kv[k] = -1;
        }
      }
      const uint64_t okm = __builtin_amdgcn_ballot_w64(ok);
      const uint32_t group = static_cast<uint32_t>(okm >> (slane & 48)) & 0xffffu;
      if (k < n && i == 0) lds_list[k] = group == 0xffffu;  // 1: the entry goes on
    }
    __syncthreads();

    for (int k = 0; k < n; ++k) {
      // every value below is workgroup-uniform (LDS), so all waves meet the barriers
      if (!__builtin_amdgcn_readfirstlane(lds_list[k])) continue;
      const int32_t rope_row = __builtin_amdgcn_readfirstlane(lds_rope[k]);
      int32_t mybt[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        mybt[b] = __builtin_amdgcn_readfirstlane(lds_ids[k][rg * NB + b]);
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
      const int tl = fresh_tid() & 63;  // epilogue addresses are recomputed per token
      merge_row_groups<RG>(lds_ml, lds_l, lds_acc, rg, half, tl, ml, l, acc);
      const int32_t t = __builtin_amdgcn_readfirstlane(lds_tok[k]);
      const int32_t kv = finish_token<kDebug, true>(p, t, rope_row, rg == 0, half, tl,
                                                    half * 256 + tl * 4, l, acc, lds_ss,
                                                    lds_stage[k]);
      if (rg == 0 && half == 0 && tl == 0) lds_kv[k] = kv;
      // No barrier here: the next token's merge writes lds_ml/l/acc only, which the epilogue
      // waves have finished reading, and its lds_ss writes follow that merge's barrier.
    }

    // ---- insert the stage's records (8-byte stores: 72 record chunks, then the scale chunk)
    __syncthreads();
    constexpr int kChunks = kSlotBytes / 8;
    for (int idx = tid; idx < n * kChunks; idx += NT) {
      const int k = idx / kChunks, c = idx - k * kChunks;
      const int32_t kv_slot = lds_kv[k];  // -1 for entries that did not go on
      if (kv_slot < 0) continue;
      const int32_t kb = kv_slot / p.kv_bs;
      const int32_t ko = kv_slot - kb * p.kv_bs;
      uint8_t* blockp = p.k_cache + static_cast<int64_t>(kb) * p.kc_stride0;
      uint8_t* dst = c < kRecordBytes / 8
                         ? blockp + static_cast<int64_t>(ko) * kRecordBytes + 8 * c
                         : blockp + static_cast<int64_t>(p.kv_bs) * kRecordBytes +
                               static_cast<int64_t>(ko) * kScaleBytes;
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(&lds_stage[k][8 * c]);
    }
    if (tid < KMAX) lds_tok[tid] = -1;  // read last by this stage's resolve
    __syncthreads();  // the next stage rewrites the stage's LDS
  }
}

}  // namespace

namespace {

// Fan-out shapes: S splits of the 16 window blocks, each streamed by RG row groups of NBW blocks.
// The workspace holds the arrival counters (kFanoutMaxTokens of them, at a fixed place so that
// calls with different T or S never overwrite a counter with partial states), then the partials.
template <int RG, int NBW>
hipError_t launch_fanout(const C128Params& p, void* ws, hipStream_t stream) {
  constexpr int S = kWindowBlocks / (RG * NBW);
  uint32_t* counters = static_cast<uint32_t*>(ws);
  float* partials = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kFanoutCounterBytes);
  const dim3 grid(static_cast<unsigned>(p.num_tokens), S);
  if (p.compressed_out)
    return launch_kernel(c128_fanout_kernel<RG, NBW, kStageRows, true>, grid, dim3(128 * RG),
                         stream, p, partials, counters);
  return launch_kernel(c128_fanout_kernel<RG, NBW, kStageRows, false>, grid, dim3(128 * RG),
                       stream, p, partials, counters);
}

}  // namespace

int fanout_auto_splits(int64_t num_tokens) {
  // Measured on MI355X (same-process timings, window sets rotated): 8 splits are fastest up to
  // 16 tokens, 4 up to 64, 2 up to 128; from about 200 tokens on the single pass already has
  // enough workgroups and the partial-state traffic makes the fan-out slower.
  if (num_tokens <= 0 || num_tokens > 128) return 1;
  if (num_tokens <= 16) return 8;
  return num_tokens <= 64 ? 4 : 2;
}

size_t fanout_workspace_bytes(int64_t num_tokens, int splits) {
  if (splits <= 1 || num_tokens <= 0 || num_tokens > kFanoutMaxTokens) return 0;
  return kFanoutCounterBytes +
         static_cast<size_t>(num_tokens) * static_cast<size_t>(splits) * 3 * kHead * sizeof(float);
}

hipError_t launch_c128_fanout(const C128Params& p, void* ws, int splits, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  if (splits > 1 && p.num_tokens > kFanoutMaxTokens) return hipErrorInvalidValue;
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
  hipError_t err = launch_kernel(c128_gate_scan_kernel, dim3(static_cast<unsigned>(nblocks)),
                                 dim3(kScanThreads), stream, p, chunk, counts, list);
  if (err != hipSuccess) return err;
  const unsigned grid =
      static_cast<unsigned>(p.num_tokens < kCompactedGrid ? p.num_tokens : kCompactedGrid);
  if (p.compressed_out)
    return launch_kernel(c128_compacted_kernel<true>, dim3(grid), dim3(128 * kRowGroups), stream,
                         p, counts, list, chunk, nblocks);
  return launch_kernel(c128_compacted_kernel<false>, dim3(grid), dim3(128 * kRowGroups), stream,
                       p, counts, list, chunk, nblocks);
}

namespace {

// Device address of `scratch` on each device, resolved with that device current on the first
// call there.  Written once under the mutex, then read without it.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* addr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!addr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    addr = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!addr) {
      err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (!addr) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(addr, std::memory_order_release);
    }
  }
  *out = addr;
  return hipSuccess;
}

}  // namespace

static_assert(kStaticCompactedScanBlocks == kMaxScanBlocks,
              "the static scratch starts with one count per scan block");

hipError_t launch_c128_compacted_static(const C128Params& p, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  if (p.num_tokens > kStaticCompactedMaxTokens) return hipErrorInvalidValue;
  if (compacted_workspace_bytes(p.num_tokens) > sizeof(scratch)) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t err = static_scratch(&ws);
  if (err != hipSuccess) return err;
  return launch_c128_compacted(p, ws, stream);
}

// Compute units of the current device (the staged grid, and the C4 kernel's wide shape, are
// sized in whole rounds of one workgroup per CU); looked up once per device, 256 on MI355X.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_c128_staged(const C128Params& p, hipStream_t stream) {
  if (p.num_tokens <= 0) return hipSuccess;
  // One round: a workgroup per CU (the LDS stage allows no second one).  Count blocks of 256
  // tokens, doubled until at most kStagedCountBlocks of them cover the batch.
  const int64_t groups = device_cu_count();
  int64_t block_tokens = 256;
  while ((p.num_tokens + block_tokens - 1) / block_tokens > kStagedCountBlocks) block_tokens *= 2;
  const int32_t nblocks = static_cast<int32_t>((p.num_tokens + block_tokens - 1) / block_tokens);
  const dim3 grid(static_cast<unsigned>(groups));
  const dim3 block(128 * kStagedRowGroups);
  if (p.compressed_out)
    return launch_kernel(
        c128_staged_kernel<kStagedRowGroups, kStageRows, kStagedWavesPerSimd, kStagedMaxTokens, true>,
        grid, block, stream, p, static_cast<int32_t>(block_tokens), nblocks);
  return launch_kernel(
      c128_staged_kernel<kStagedRowGroups, kStageRows, kStagedWavesPerSimd, kStagedMaxTokens, false>,
      grid, block, stream, p, static_cast<int32_t>(block_tokens), nblocks);
}

}  // namespace dsv4
