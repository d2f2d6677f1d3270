// Read-bandwidth reference kernels for the bench (not part of the C128 library).
//
//  * stream_read: every lane streams 16-byte vectors through a grid-stride loop
//    with 8 loads in flight, summing them (a plain sequential read of a buffer).
//  * block_gather_read: workgroup w reads the 16 state blocks listed in
//    ids[16w .. 16w+15] (32 KiB each when stride0 = 8192 floats) with the same
//    lane-to-16-byte-vector mapping as the compress kernel, summing them: the
//    compress kernel's exact HBM access pattern without its arithmetic.
// Each comes with plain loads and with the non-temporal hint the compress kernels use.
// Both write one float per workgroup so the loads cannot be removed.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

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

}  // namespace

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
