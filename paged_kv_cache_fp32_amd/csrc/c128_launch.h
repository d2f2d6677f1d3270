// Host-side launchers of the C128 compress-store kernels (internal; the C ABI in c128_abi.cpp
// validates the arguments and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

#include "c128_params.h"

namespace dsv4 {

// Launch `kernel` on `stream` and return the status of this launch alone.  (hipGetLastError after
// a <<<>>> launch would also report, and clear, an earlier error of the calling thread.)  The
// arguments are converted to the kernel's parameter types before their addresses are taken.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                         A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  std::tuple<std::decay_t<P>...> vals(std::forward<A>(args)...);
  return std::apply(
      [&](auto&... v) {
        void* argv[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0,
                               stream);
      },
      vals);
}

// Single pass and encoder: c128_kernel.hip.  Every launcher returns the hipError_t of its launch.
// Batches of kStagedMinTokens and more go to the staged schedule.
hipError_t launch_c128_compress_store(const C128Params& p, hipStream_t stream);
// Staged schedule for large batches (c128_schedules.hip): one workgroup of kStagedRowGroups row
// groups per CU takes an equal share of the tokens that pass the gate and streams it in stages
// of up to kStagedMaxTokens tokens, inserting a stage's records after its last state read.
constexpr int64_t kStagedMinTokens = 2048;
constexpr int kStagedMaxTokens = 64;
constexpr int kStagedRowGroups = 8;
constexpr int kStagedWavesPerSimd = 4;
hipError_t launch_c128_staged(const C128Params& p, hipStream_t stream);
// Fan-out and compacted schedules: c128_schedules.hip.
// Fan-out over `splits` workgroups per token (1, 2, 4, 8 or 16; 1 is the single pass) for at
// most kFanoutMaxTokens tokens, with a workspace of fanout_workspace_bytes(T, splits) bytes,
// 16-byte aligned, whose first kFanoutCounterBytes (the per-token arrival counters) are zero
// before the call; the call leaves them zero.
constexpr int64_t kFanoutMaxTokens = 4096;
constexpr size_t kFanoutCounterBytes = kFanoutMaxTokens * sizeof(uint32_t);
hipError_t launch_c128_fanout(const C128Params& p, void* ws, int splits, hipStream_t stream);
int fanout_auto_splits(int64_t num_tokens);
size_t fanout_workspace_bytes(int64_t num_tokens, int splits);
// Compacted schedule for long varlen batches: a gate scan into a workspace of
// compacted_workspace_bytes(T) bytes (16-byte aligned), then a persistent grid over the tokens
// that pass.
hipError_t launch_c128_compacted(const C128Params& p, void* ws, hipStream_t stream);
size_t compacted_workspace_bytes(int64_t num_tokens);
// The same schedule with its counts and token list in a fixed device array of the library (no
// workspace, no allocation), for at most kStaticCompactedMaxTokens tokens.  Calls that overlap
// on one device share the array and race.
constexpr int kStaticCompactedScanBlocks = 1024;
constexpr int64_t kStaticCompactedMaxTokens = int64_t(1) << 20;
hipError_t launch_c128_compacted_static(const C128Params& p, hipStream_t stream);
// C4 compressor (ratio 4, overlapping 8-row window), one wave per token: c4_kernel.hip.
// state_bs is the state cache's rows per block.
// Compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_c4_compress_store(const C128Params& p, int32_t state_bs, hipStream_t stream);
// Indexer FP8 compressor (head 128, ratio 4, overlapping window): indexer_kernel.hip.
hipError_t launch_indexer_compress_store(const C128Params& p, int32_t state_bs,
                                         hipStream_t stream);
// The same compressor with the MXFP4 cache, and its E2M1 encoder on an array: indexer_kernel.hip.
hipError_t launch_indexer_mxfp4_compress_store(const C128Params& p, int32_t state_bs,
                                               hipStream_t stream);
hipError_t launch_e2m1_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream);
hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

}  // namespace dsv4
