// Read-bandwidth reference kernels for the bench (not part of the C128 library).
//
//  * stream_read: every lane streams 16-byte vectors through a grid-stride loop
//    with 8 loads in flight, summing them (a plain sequential read of a buffer).
//  * block_gather_read: workgroup w reads the 16 state blocks listed in
//    ids[16w .. 16w+15] (32 KiB each when stride0 = 8192 floats) with the same
//    lane-to-16-byte-vector mapping as the compress kernel, summing them: the
//    compress kernel's exact HBM access pattern without its arithmetic.
//  * stream_chunks: a sequential read in contiguous chunks per workgroup.
//  * window_read_split: small batches' windows read with S workgroups per window.
//  * idx_window_read: the indexer and C4 compressors' reads (metadata, 8 half-rows, RoPE row).
//  * window_read_persistent: large batches' windows read by a persistent grid of any shape.
// The first three come with plain loads and with the non-temporal hint the compress kernels
// use. Each writes one float per workgroup or wave so the loads cannot be removed.

#include <hip/hip_runtime.h>
#include <stdint.h>

struct IdxProbe {
  const float* pool;
  int64_t s0, s1;  // floats per pool block, per row
  const int32_t* positions;
  const int32_t* slot;
  const int32_t* req;
  const int32_t* bt;
  int64_t bt_stride;
  int32_t bt_rows, bt_cols, n_blocks;
  const int64_t* offs;  // mode 1: [T][8] row offsets in floats, -1 for a row not read
  const float* cs;
  int64_t cs_stride;
  int32_t cs_rows;
  int32_t T, kpw;
  uint32_t nb_mask;     // mode 2: pool blocks - 1 (a power of two minus one)
};

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <bool kNt>
__device__ __forceinline__ float4 ld(const float4* p) {
  if constexpr (kNt) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

template <bool kNt>
__global__ void __launch_bounds__(512) stream_read(const float4* __restrict__ p, int64_t n4,
                                                   float* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  float acc = 0.0f;
  for (; i + 7 * stride < n4; i += 8 * stride) {
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = ld<kNt>(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (v[k].x + v[k].y) + (v[k].z + v[k].w);
  }
  for (; i < n4; i += stride) {
    const float4 v = ld<kNt>(p + i);
    acc += (v.x + v.y) + (v.z + v.w);
  }
  if (threadIdx.x == 0 || acc == 1234.5f) out[blockIdx.x] = acc;
}

// Sequential read in contiguous chunks: workgroup w reads chunks w, w + G, ... of U * blockDim.x
// 16-byte vectors each (U loads per lane, all issued before any is summed).  Consecutive lanes
// read consecutive vectors, so every wave-wide load is 1 KiB contiguous and a chunk is one
// contiguous range (32 KiB to 128 KiB).  n4 is a multiple of the chunk size (checked on the host).
template <int U, bool kNt>
__global__ void __launch_bounds__(512) stream_chunks(const float4* __restrict__ p, int64_t n4,
                                                     float* __restrict__ out) {
  const int64_t chunk4 = static_cast<int64_t>(U) * blockDim.x;
  float acc = 0.0f;
  for (int64_t c = blockIdx.x; (c + 1) * chunk4 <= n4; c += gridDim.x) {
    const float4* base = p + c * chunk4 + threadIdx.x;
    float4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = ld<kNt>(base + k * blockDim.x);
#pragma unroll
    for (int k = 0; k < U; ++k) acc += (v[k].x + v[k].y) + (v[k].z + v[k].w);
  }
  if (threadIdx.x == 0 || acc == 1234.5f) out[blockIdx.x] = acc;
}

// 512 lanes: lane l of wave w covers 16-byte vector (w % 2) * 64 + l of each 4 KiB row
// half pair ... here simply: the workgroup sweeps each 32 KiB block with 512 x 16 B per step.
template <bool kNt>
__global__ void __launch_bounds__(512) block_gather_read(const float* __restrict__ pool,
                                                         int64_t stride0,
                                                         const int32_t* __restrict__ ids,
                                                         float* __restrict__ out) {
  const int32_t* my = ids + static_cast<int64_t>(blockIdx.x) * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int half = wave & 1, rg = wave >> 1;  // 2 column halves x 4 row groups, as the kernel
  const int col = half * 256 + lane * 4;
  float acc = 0.0f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float* base = pool + static_cast<int64_t>(my[rg * 4 + b]) * stride0 + col;
    float4 v[16];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      v[2 * r] = ld<kNt>(reinterpret_cast<const float4*>(base + r * 1024));
      v[2 * r + 1] = ld<kNt>(reinterpret_cast<const float4*>(base + r * 1024 + 512));
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) acc += (v[k].x + v[k].y) + (v[k].z + v[k].w);
  }
  if (threadIdx.x == 0 || acc == 1234.5f) out[blockIdx.x] = acc;
}

// The window gather of small batches, split: token t's window is 16 blocks x 8 rows x 4
// quarter-rows of 1 KiB (kv left / right, score left / right) = 512 pieces.  Workgroup (t, s)
// of S per token has W waves; wave w reads a contiguous range of 512 / (S * W) pieces, L one-KiB
// wave loads in flight at a time (non-temporal, as the compress kernels load).
template <int L>
__global__ void __launch_bounds__(1024) window_read_split(const float* __restrict__ pool,
                                                          int64_t stride0,
                                                          const int32_t* __restrict__ ids,
                                                          int S, int W, float* __restrict__ out) {
  const int t = blockIdx.x, s = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = 512 / (S * W);
  const int p0 = s * (512 / S) + wave * n;
  const int32_t* my = ids + static_cast<int64_t>(t) * 16;
  float acc = 0.0f;
  for (int k = 0; k < n; k += L) {
    float4 v[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int p = p0 + k + j;
      const int b = p >> 5, q = p & 31, r = q >> 2, part = q & 3;
      const float* a = pool + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(my[b])) * stride0 +
                       r * 1024 + (part >> 1) * 512 + (part & 1) * 256 + lane * 4;
      v[j] = ld<true>(reinterpret_cast<const float4*>(a));
    }
#pragma unroll
    for (int j = 0; j < L; ++j) acc += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  }
  if (threadIdx.x == 0 || acc == 1234.5f) out[t * S + s] = acc;
}


// The window gather of large batches by a persistent grid: workgroup g reads windows g, g + G,
// ...; a window is 16 blocks x 8 rows x 4 quarter-rows of 1 KiB = 512 pieces, split evenly over
// the workgroup's W waves, each keeping L one-KiB wave loads in flight (non-temporal, as the
// compress kernels load).  Its launch shape is free, unlike the compress kernels'.
template <int L>
__global__ void __launch_bounds__(1024) window_read_persistent(const float* __restrict__ pool,
                                                               int64_t stride0,
                                                               const int32_t* __restrict__ ids,
                                                               int n_windows, int W,
                                                               float* __restrict__ out) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = 512 / W;
  float acc = 0.0f;
  for (int w = blockIdx.x; w < n_windows; w += gridDim.x) {
    const int32_t* my = ids + static_cast<int64_t>(w) * 16;
    for (int k = 0; k < n; k += L) {
      float4 v[L];
#pragma unroll
      for (int j = 0; j < L; ++j) {
        const int p = wave * n + k + j;
        const int b = p >> 5, q = p & 31;  // block; row q >> 2, quarter q & 3
        const float* a = pool +
                         static_cast<int64_t>(__builtin_amdgcn_readfirstlane(my[b])) * stride0 +
                         q * 256 + lane * 4;
        v[j] = ld<true>(reinterpret_cast<const float4*>(a));
      }
#pragma unroll
      for (int j = 0; j < L; ++j) acc += (v[j].x + v[j].y) + (v[j].z + v[j].w);
    }
  }
  if (threadIdx.x == 0 || acc == 1234.5f) out[blockIdx.x] = acc;
}


// The indexer or C4 compressor's reads without its arithmetic or its record stores.  A wave
// takes kpw consecutive tokens; lane (k, i) = (lane / 8, lane % 8) resolves window row i of
// token k; per token the wave loads the 8 half-rows (indexer: 512 B of kv and 512 B of score
// each; C4: 2 KiB of each) and the RoPE row, non-temporal, and sums them.
//  mode 0: gate, request and block ids read as the compressor reads them (positions,
//          slot_mapping, token_to_req, then the block table: two dependent round trips);
//  mode 1: the row offsets precomputed on the host (one round trip: offs and positions);
//  mode 2: no metadata: token t reads rows 0..7 of pool block (t * 2654435761) & nb_mask.

template <int kMode, bool kC4>
__global__ void __launch_bounds__(256) idx_window_read(const IdxProbe p, float* __restrict__ out) {
  // head 128 (indexer): a row is kv 2 x 128 | score 2 x 128, lane l loads 8 bytes at column 2l
  // of each half-row; head 512 (C4): kv 2 x 512 | score 2 x 512, lane l loads 16 bytes at
  // columns 4l and 256 + 4l of each half-row
  constexpr int kHalf = kC4 ? 512 : 128;      // floats in the kv (or score) half of a row
  constexpr int kScore = 2 * kHalf;           // score part of a row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const int64_t tbase = wid * p.kpw;
  const int mk = lane >> 3, mi = lane & 7;
  const int64_t mt = tbase + mk;
  int64_t moff = -1;
  int32_t mrow = -1;  // RoPE row
  if (mk < p.kpw && mt < p.T) {
    if constexpr (kMode == 0) {
      const int32_t pos = p.positions[mt], s = p.slot[mt], r = p.req[mt];
      if (s >= 0 && pos >= 0 && (pos & 3) == 3 && r >= 0 && r < p.bt_rows) {
        const int32_t q = pos - 7 + mi;
        if (q >= 0 && (q >> 3) < p.bt_cols) {
          const int32_t b = p.bt[static_cast<int64_t>(r) * p.bt_stride + (q >> 3)];
          if (static_cast<uint32_t>(b) < static_cast<uint32_t>(p.n_blocks))
            moff = b * p.s0 + (q & 7) * p.s1 + (mi >= 4 ? kHalf : 0);
        }
        mrow = pos & ~3;
      }
    } else if constexpr (kMode == 1) {
      moff = p.offs[mt * 8 + mi];
      mrow = p.positions[mt] & ~3;
    } else {
      const uint32_t b = static_cast<uint32_t>(mt * 2654435761ull) & p.nb_mask;
      moff = b * p.s0 + mi * p.s1 + (mi >= 4 ? kHalf : 0);
      mrow = static_cast<int32_t>(mt & 1023) * 4;
    }
    if (mrow >= p.cs_rows) mrow = -1;
  }
  float acc = 0.0f;
  for (int k = 0; k < p.kpw; ++k) {
    int64_t off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(moff), 8 * k + i);
      const uint32_t hi = __builtin_amdgcn_readlane(
          static_cast<uint32_t>(static_cast<uint64_t>(moff) >> 32), 8 * k + i);
      off[i] = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    }
    const int32_t row = __builtin_amdgcn_readlane(mrow, 8 * k);
    if constexpr (kC4) {
      float4 v[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (off[i] >= 0) {
          const float* r = p.pool + off[i] + 4 * lane;
          v[i][0] = ld<true>(reinterpret_cast<const float4*>(r));
          v[i][1] = ld<true>(reinterpret_cast<const float4*>(r + 256));
          v[i][2] = ld<true>(reinterpret_cast<const float4*>(r + kScore));
          v[i][3] = ld<true>(reinterpret_cast<const float4*>(r + kScore + 256));
        } else {
          v[i][0] = v[i][1] = v[i][2] = v[i][3] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      float4 c = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row >= 0) {
        const float* cs = p.cs + static_cast<int64_t>(row) * p.cs_stride;
        const int j = lane & 15;
        c = make_float4(cs[2 * j], cs[2 * j + 1], cs[32 + 2 * j], cs[33 + 2 * j]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int h = 0; h < 4; ++h) acc += (v[i][h].x + v[i][h].y) + (v[i][h].z + v[i][h].w);
      acc += (c.x + c.y) + (c.z + c.w);
    } else {
      float2 v[17];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (off[i] >= 0) {
          const f32x2 a = __builtin_nontemporal_load(
              reinterpret_cast<const f32x2*>(p.pool + off[i] + 2 * lane));
          const f32x2 b = __builtin_nontemporal_load(
              reinterpret_cast<const f32x2*>(p.pool + off[i] + kScore + 2 * lane));
          v[2 * i] = make_float2(a.x, a.y);
          v[2 * i + 1] = make_float2(b.x, b.y);
        } else {
          v[2 * i] = v[2 * i + 1] = make_float2(0.f, 0.f);
        }
      }
      v[16] = make_float2(0.f, 0.f);
      if (row >= 0 && lane >= 32) {
        const float* c = p.cs + static_cast<int64_t>(row) * p.cs_stride;
        v[16] = make_float2(c[lane - 32], c[lane]);
      }
#pragma unroll
      for (int j = 0; j < 17; ++j) acc += v[j].x + v[j].y;
    }
  }
  if (lane == 0 || acc == 1234.5f) out[wid] = acc;
}
}  // namespace

// Split window gather of `n_windows` windows (ids: 16 block ids each; pool blocks of 8 rows of
// 1024 floats at stride0 >= 8192 floats): S in {1, 2, 4, 8} workgroups per window, W in {4, 8, 16}
// waves, L in {4, 8, 16, 32} loads in flight with L dividing 512 / (S * W); out holds
// n_windows * S floats.
extern "C" int probe_window_read_split(const float* pool, int64_t stride0, const int32_t* ids,
                                       int n_windows, int S, int W, int L, float* out,
                                       void* stream) {
  if (!pool || !ids || !out || n_windows < 1 || stride0 < 8192) return -1;
  if ((S != 1 && S != 2 && S != 4 && S != 8) || (W != 4 && W != 8 && W != 16)) return -1;
  const int n = 512 / (S * W);
  if (L > n || n % L) return -1;
  const dim3 grid(n_windows, S), block(64 * W);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (L) {
    case 4: window_read_split<4><<<grid, block, 0, st>>>(pool, stride0, ids, S, W, out); break;
    case 8: window_read_split<8><<<grid, block, 0, st>>>(pool, stride0, ids, S, W, out); break;
    case 16: window_read_split<16><<<grid, block, 0, st>>>(pool, stride0, ids, S, W, out); break;
    case 32: window_read_split<32><<<grid, block, 0, st>>>(pool, stride0, ids, S, W, out); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// Persistent window gather of `n_windows` windows (ids: 16 block ids each; pool blocks of 8 rows of
// 1024 floats at stride0 >= 8192 floats) by G workgroups of W in {2, 4, 8, 16} waves, L in
// {4, 8, 16} loads in flight per lane with L dividing 512 / W; out holds G floats.
extern "C" int probe_window_read_persistent(const float* pool, int64_t stride0,
                                            const int32_t* ids, int n_windows, int G, int W,
                                            int L, float* out, void* stream) {
  if (!pool || !ids || !out || n_windows < 1 || G < 1 || stride0 < 8192) return -1;
  if (W != 2 && W != 4 && W != 8 && W != 16) return -1;
  if ((L != 4 && L != 8 && L != 16) || (512 / W) % L) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(G), block(64 * W);
  switch (L) {
    case 4:
      window_read_persistent<4><<<grid, block, 0, st>>>(pool, stride0, ids, n_windows, W, out);
      break;
    case 8:
      window_read_persistent<8><<<grid, block, 0, st>>>(pool, stride0, ids, n_windows, W, out);
      break;
    default:
      window_read_persistent<16><<<grid, block, 0, st>>>(pool, stride0, ids, n_windows, W, out);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

extern "C" int probe_stream_read(const void* p, int64_t bytes, float* out, int blocks,
                                 int threads, int nt, void* stream) {
  if (!p || !out || bytes < 16 || blocks < 1 || threads < 64 || threads > 512) return -1;
  if (nt)
    stream_read<true><<<blocks, threads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const float4*>(p), bytes / 16, out);
  else
    stream_read<false><<<blocks, threads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const float4*>(p), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

extern "C" int probe_block_gather_read(const float* pool, int64_t stride0, const int32_t* ids,
                                       int n_windows, float* out, int nt, void* stream) {
  if (!pool || !ids || !out || n_windows < 1 || stride0 < 8192) return -1;
  if (nt)
    block_gather_read<true><<<n_windows, 512, 0, static_cast<hipStream_t>(stream)>>>(
        pool, stride0, ids, out);
  else
    block_gather_read<false><<<n_windows, 512, 0, static_cast<hipStream_t>(stream)>>>(
        pool, stride0, ids, out);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

namespace {
template <int U>
int launch_chunks(const void* p, int64_t n4, float* out, int blocks, int threads, int nt,
                  hipStream_t stream) {
  if (nt)
    stream_chunks<U, true><<<blocks, threads, 0, stream>>>(static_cast<const float4*>(p), n4, out);
  else
    stream_chunks<U, false><<<blocks, threads, 0, stream>>>(static_cast<const float4*>(p), n4, out);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
}  // namespace

// Sequential chunked read of `bytes` (a multiple of loads * threads * 16) by `blocks`
// workgroups of `threads` lanes, `loads` 16-byte loads per lane per chunk (4, 8 or 16).
extern "C" int probe_stream_chunks(const void* p, int64_t bytes, float* out, int blocks,
                                   int threads, int loads, int nt, void* stream) {
  if (!p || !out || blocks < 1 || threads < 64 || threads > 512 || threads % 64) return -1;
  const int64_t chunk = static_cast<int64_t>(loads) * threads * 16;
  if (bytes < chunk || bytes % chunk) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (loads) {
    case 4: return launch_chunks<4>(p, bytes / 16, out, blocks, threads, nt, s);
    case 8: return launch_chunks<8>(p, bytes / 16, out, blocks, threads, nt, s);
    case 16: return launch_chunks<16>(p, bytes / 16, out, blocks, threads, nt, s);
    default: return -1;
  }
}

// Window reads of the indexer compressor (head 128) or of the C4 compressor (head 512) with
// the kernel's lane mapping (idx_window_read above): p.T tokens, p.kpw (1..8) per wave, 4 waves
// a workgroup; out holds one float per wave.
namespace {
template <bool kC4>
int launch_window_read(const IdxProbe* p, int mode, float* out, void* stream) {
  if (!p || !out || !p->pool || p->T < 1 || p->kpw < 1 || p->kpw > 8 || !p->cs) return -1;
  if (mode == 0 && (!p->positions || !p->slot || !p->req || !p->bt)) return -1;
  if (mode == 1 && (!p->offs || !p->positions)) return -1;
  if (mode == 2 && ((p->nb_mask + 1u) & p->nb_mask) != 0) return -1;
  const int64_t waves = (static_cast<int64_t>(p->T) + p->kpw - 1) / p->kpw;
  const dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: idx_window_read<0, kC4><<<grid, block, 0, st>>>(*p, out); break;
    case 1: idx_window_read<1, kC4><<<grid, block, 0, st>>>(*p, out); break;
    case 2: idx_window_read<2, kC4><<<grid, block, 0, st>>>(*p, out); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
}  // namespace

extern "C" int probe_indexer_window_read(const IdxProbe* p, int mode, float* out, void* stream) {
  return launch_window_read<false>(p, mode, out, stream);
}

extern "C" int probe_c4_window_read(const IdxProbe* p, int mode, float* out, void* stream) {
  return launch_window_read<true>(p, mode, out, stream);
}
