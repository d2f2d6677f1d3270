// Layout constants and launch parameters of the C128 compress-store kernels (not part of the
// public ABI; include/dsv4_c128.h holds the contract).
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

}  // namespace dsv4
