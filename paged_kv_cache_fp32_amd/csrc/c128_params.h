// Internal launch parameters of the C128 compress-store kernel (not part of
// the public ABI; see include/dsv4_c128.h for the contract).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv4 {

// Fixed by the DeepSeek-V4 C128 layout (vLLM PR 44230, "Summary"; vLLM
// fused_compress_quant_cache page, sparse-attention kernel constants).
constexpr int kHead = 512;         // head size = state width
constexpr int kNope = 448;         // FP8 dims
constexpr int kRope = 64;          // bf16 RoPE dims
constexpr int kRatio = 128;        // compress ratio: rows per window
constexpr int kStateBlock = 8;     // state-cache block size
constexpr int kWindowBlocks = kRatio / kStateBlock;  // 16 blocks per window
constexpr int kRowFloats = 2 * kHead;                // kv | score
constexpr int kQuantBlock = 64;
constexpr int kNumQuant = kNope / kQuantBlock;       // 7
constexpr int kRecordBytes = 576;  // 448 fp8 + 64 bf16
constexpr int kScaleBytes = 8;     // 7 UE8M0 + 1 zero pad
constexpr int kSlotBytes = kRecordBytes + kScaleBytes;  // 584

struct C128Params {
  const float* state;      // [S, 8, 1024] fp32
  int64_t s0, s1;          // element strides of block and row
  int32_t n_state_blocks;  // S
  const int32_t* block_table;
  int64_t bt_stride;       // elements
  int32_t bt_rows, bt_cols;
  const int32_t* token_to_req;
  const int32_t* positions;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  const float* rms_w;
  float eps;
  const float* cos_sin;
  int64_t cs_stride;       // elements
  int32_t cs_rows;
  uint8_t* k_cache;
  int64_t kc_stride0;      // bytes
  int32_t kv_bs;
  int64_t n_kv_slots;      // B * bs
  const int32_t* kv_slot_mapping;
  float* compressed_out;   // [T, 512] or nullptr
};

// Launchers (c128_kernel.hip).  Return the hipError_t of the launch.
hipError_t launch_c128_compress_store(const C128Params& p, hipStream_t stream);
// Fan-out over `splits` workgroups per token (1, 2, 4, 8 or 16; 1 is the single pass) with a
// workspace of fanout_workspace_bytes(T, splits) bytes, 16-byte aligned.
hipError_t launch_c128_fanout(const C128Params& p, float* ws, int splits, hipStream_t stream);
int fanout_auto_splits(int64_t num_tokens);
size_t fanout_workspace_bytes(int64_t num_tokens, int splits);
// Compacted schedule for long varlen batches: a gate scan into a workspace of
// compacted_workspace_bytes(T) bytes (16-byte aligned), then a persistent grid over the tokens
// that pass.
hipError_t launch_c128_compacted(const C128Params& p, void* ws, hipStream_t stream);
size_t compacted_workspace_bytes(int64_t num_tokens);
hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

}  // namespace dsv4
