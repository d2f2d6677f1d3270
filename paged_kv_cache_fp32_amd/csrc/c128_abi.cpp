// C ABI of the compress-store library (C128, C4, indexer FP8): descriptor validation
// (host only), launch, error codes and the per-thread error message.  The
// contract is documented in include/dsv4_c128.h.
//
// The validation mirrors the layout limits of the DeepSeek-V4 C128 path
// (vLLM PR 44230, "Summary" and "Changes": head 512, state width 512,
// compress ratio 128, state block 8, KV block size taken from
// k_cache.shape[1]; the wrapper rejects unsupported layouts up front) and
// the argument list of the page's launcher `compress_norm_rope_store_triton`
// (block table row stride, cos/sin row stride, k_cache.stride(0) as the
// block stride in bytes).

#include <cstdarg>
#include <cstdio>
#include <string>

#include "c128_launch.h"
#include "dsv4_c128.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

constexpr int64_t kI32Max = 2147483647;
// Largest span of a tensor, first to last element, in bytes: far beyond any device
// allocation, and small enough that no index times stride the kernels form can overflow
// 64-bit address arithmetic.
constexpr int64_t kMaxSpanBytes = int64_t(1) << 48;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_tensor(const dsv4_tensor* t, const char* name, int dtype, int ndim) {
  if (!t) return fail(DSV4_ERR_NULL, "%s: descriptor is NULL", name);
  if (t->ndim != ndim)
    return fail(DSV4_ERR_RANK, "%s: expected %d dimensions, got %d", name, ndim, t->ndim);
  if (t->dtype != dtype)
    return fail(DSV4_ERR_DTYPE, "%s: wrong dtype code %d (expected %d)", name, t->dtype, dtype);
  for (int d = 0; d < ndim; ++d) {
    if (t->shape[d] < 0 || t->shape[d] > kI32Max)
      return fail(DSV4_ERR_SHAPE, "%s: shape[%d] = %lld out of range", name, d,
                  static_cast<long long>(t->shape[d]));
  }
  int64_t numel = 1;
  for (int d = 0; d < ndim; ++d) numel *= t->shape[d];
  if (numel > 0 && !t->data) return fail(DSV4_ERR_NULL, "%s: data pointer is NULL", name);
  // strides of dimensions longer than 1: non-negative, and a span below kMaxSpanBytes
  const int64_t esize = dtype == DSV4_U8 ? 1 : 4;
  int64_t span = 0;
  for (int d = 0; d < ndim; ++d) {
    if (t->shape[d] <= 1) continue;
    if (t->stride[d] < 0)
      return fail(DSV4_ERR_STRIDE, "%s: stride[%d] = %lld is negative", name, d,
                  static_cast<long long>(t->stride[d]));
    if (t->stride[d] > kMaxSpanBytes / esize / (t->shape[d] - 1) ||
        (span += (t->shape[d] - 1) * t->stride[d] * esize) > kMaxSpanBytes)
      return fail(DSV4_ERR_STRIDE, "%s: the strides span more than 2^48 bytes", name);
  }
  return DSV4_OK;
}

int check_token_array(const dsv4_tensor* t, const char* name, int64_t T) {
  int rc = check_tensor(t, name, DSV4_I32, 1);
  if (rc) return rc;
  if (t->shape[0] != T)
    return fail(DSV4_ERR_SHAPE, "%s: length %lld differs from positions (%lld)", name,
                static_cast<long long>(t->shape[0]), static_cast<long long>(T));
  if (T > 1 && t->stride[0] != 1)
    return fail(DSV4_ERR_STRIDE, "%s: must be contiguous (stride %lld)", name,
                static_cast<long long>(t->stride[0]));
  return DSV4_OK;
}

// Layout a compressor expects: state row width in floats, rows per block (0 = any positive
// count), the fewest block-table columns a window can need, the head size (rms_w length), the
// cache's bytes per token (last k_cache dimension) and the alignment its stores need.
struct StateLayout {
  const char* path;
  int64_t row_floats;
  int64_t block_rows;
  int64_t min_bt_cols;
  int64_t head;
  int64_t slot_bytes;
  int64_t kc_align;
};
// C128: kv 512 | score 512, blocks of 8 rows, 16 blocks per window; 576 + 8 cache bytes.
constexpr StateLayout kC128Layout{"C128", dsv4::kRowFloats, dsv4::kStateBlock,
                                  dsv4::kWindowBlocks, dsv4::kHead, dsv4::kSlotBytes, 8};
// C4 with its overlapping window: kv 2 x 512 | score 2 x 512; any block size.
constexpr StateLayout kC4Layout{"C4", 4 * dsv4::kHead, 0, 1, dsv4::kHead, dsv4::kSlotBytes, 8};
// Indexer (head 128, overlapping window of ratio 4): kv 2 x 128 | score 2 x 128; 128 fp8
// bytes + one fp32 scale per token.
constexpr StateLayout kIndexerLayout{"indexer", 4 * 128, 0, 1, 128, 128 + 4, 4};
// The same with the MXFP4 cache: 64 bytes of E2M1 codes + 4 UE8M0 bytes per token.
constexpr StateLayout kIndexerMxfp4Layout{"indexer MXFP4", 4 * 128, 0, 1, 128, 64 + 4, 4};

int validate_all(const dsv4_tensor* state, const dsv4_tensor* bt, const dsv4_tensor* t2r,
                 const dsv4_tensor* pos, const dsv4_tensor* slot, const dsv4_tensor* w, float eps,
                 const dsv4_tensor* cs, const dsv4_tensor* kc, const dsv4_tensor* kvs,
                 dsv4::C128Params* out, const StateLayout& L = kC128Layout,
                 int32_t* state_bs = nullptr) {
  using namespace dsv4;
  int rc;
  // positions defines T; every other token array must match it
  if ((rc = check_tensor(pos, "positions", DSV4_I32, 1))) return rc;
  const int64_t T = pos->shape[0];
  if (T > DSV4_MAX_TOKENS)
    return fail(DSV4_ERR_SHAPE, "positions: %lld tokens, at most %lld per call",
                static_cast<long long>(T), static_cast<long long>(DSV4_MAX_TOKENS));
  if ((rc = check_token_array(pos, "positions", T))) return rc;
  if ((rc = check_token_array(t2r, "token_to_req", T))) return rc;
  if ((rc = check_token_array(slot, "slot_mapping", T))) return rc;
  if ((rc = check_token_array(kvs, "kv_slot_mapping", T))) return rc;

  // state cache f32 [S, rows per block, row floats]
  if ((rc = check_tensor(state, "state_cache", DSV4_F32, 3))) return rc;
  const int64_t sbs = state->shape[1];
  if (L.block_rows ? sbs != L.block_rows : sbs < 1)
    return fail(DSV4_ERR_SHAPE, "state_cache: block size %lld, the %s path needs %s",
                static_cast<long long>(sbs), L.path, L.block_rows ? "8" : ">= 1");
  if (state->shape[2] != L.row_floats)
    return fail(DSV4_ERR_SHAPE, "state_cache: row of %lld floats, the %s path needs %lld",
                static_cast<long long>(state->shape[2]), L.path,
                static_cast<long long>(L.row_floats));
  if (state->stride[2] != 1) return fail(DSV4_ERR_STRIDE, "state_cache: stride[2] must be 1");
  if (state->stride[1] < L.row_floats)
    return fail(DSV4_ERR_STRIDE, "state_cache: stride[1] = %lld < %lld (rows overlap)",
                static_cast<long long>(state->stride[1]), static_cast<long long>(L.row_floats));
  if (sbs > 1 ? state->stride[0] < sbs * state->stride[1] : state->stride[0] < L.row_floats)
    return fail(DSV4_ERR_STRIDE, "state_cache: stride[0] = %lld too small (blocks overlap)",
                static_cast<long long>(state->stride[0]));
  if (!aligned16(state->data) || (state->stride[1] & 3) || (state->stride[0] & 3))
    return fail(DSV4_ERR_ALIGN, "state_cache: data and strides must be 16-byte aligned");

  // block table i32 [R, M]
  if ((rc = check_tensor(bt, "block_table", DSV4_I32, 2))) return rc;
  if (bt->shape[1] < L.min_bt_cols)
    return fail(DSV4_ERR_SHAPE, "block_table: %lld columns, a %s window needs %lld",
                static_cast<long long>(bt->shape[1]), L.path,
                static_cast<long long>(L.min_bt_cols));
  if (bt->stride[1] != 1) return fail(DSV4_ERR_STRIDE, "block_table: stride[1] must be 1");
  if (bt->shape[0] > 1 && bt->stride[0] < bt->shape[1])
    return fail(DSV4_ERR_STRIDE, "block_table: stride[0] < shape[1] (rows overlap)");

  // rms weight f32 [512]
  if ((rc = check_tensor(w, "rms_w", DSV4_F32, 1))) return rc;
  if (w->shape[0] != L.head)
    return fail(DSV4_ERR_SHAPE, "rms_w: %lld entries, the %s head size is %lld",
                static_cast<long long>(w->shape[0]), L.path, static_cast<long long>(L.head));
  if (w->stride[0] != 1) return fail(DSV4_ERR_STRIDE, "rms_w: must be contiguous");
  if (!aligned16(w->data)) return fail(DSV4_ERR_ALIGN, "rms_w: data must be 16-byte aligned");
  if (!(eps >= 0.0f) || eps != eps)
    return fail(DSV4_ERR_SHAPE, "eps must be a non-negative number");

  // cos/sin f32 [P, >=64]
  if ((rc = check_tensor(cs, "cos_sin", DSV4_F32, 2))) return rc;
  if (cs->shape[1] < kRope)
    return fail(DSV4_ERR_SHAPE, "cos_sin: %lld columns, RoPE needs 64 (cos 32 | sin 32)",
                static_cast<long long>(cs->shape[1]));
  if (cs->stride[1] != 1) return fail(DSV4_ERR_STRIDE, "cos_sin: stride[1] must be 1");
  if (cs->shape[0] > 1 && cs->stride[0] < cs->shape[1])
    return fail(DSV4_ERR_STRIDE, "cos_sin: stride[0] < shape[1] (rows overlap)");

  // k_cache u8 [B, bs, slot bytes]: 584 (576 data + 8 scale) or, for the indexer, 132
  if ((rc = check_tensor(kc, "k_cache", DSV4_U8, 3))) return rc;
  if (kc->shape[2] != L.slot_bytes)
    return fail(DSV4_ERR_SHAPE, "k_cache: last dimension %lld, the %s cache layout needs %lld "
                "bytes per token", static_cast<long long>(kc->shape[2]), L.path,
                static_cast<long long>(L.slot_bytes));
  if (kc->shape[1] < 1) return fail(DSV4_ERR_SHAPE, "k_cache: block size must be >= 1");
  if (kc->stride[2] != 1 || kc->stride[1] != L.slot_bytes)
    return fail(DSV4_ERR_STRIDE, "k_cache: stride[2] must be 1 and stride[1] %lld",
                static_cast<long long>(L.slot_bytes));
  if (kc->stride[0] < kc->shape[1] * L.slot_bytes)
    return fail(DSV4_ERR_STRIDE, "k_cache: stride[0] = %lld < bs*%lld = %lld",
                static_cast<long long>(kc->stride[0]), static_cast<long long>(L.slot_bytes),
                static_cast<long long>(kc->shape[1] * L.slot_bytes));
  // records are stored with 4- or 8-byte stores (bs*584 is a multiple of 8, bs*132 of 4)
  if ((reinterpret_cast<uintptr_t>(kc->data) & (L.kc_align - 1)) ||
      (kc->stride[0] & (L.kc_align - 1)))
    return fail(DSV4_ERR_ALIGN, "k_cache: data and stride[0] must be %lld-byte aligned",
                static_cast<long long>(L.kc_align));

  if (out) {
    out->state = static_cast<const float*>(state->data);
    out->s0 = state->stride[0];
    out->s1 = state->stride[1];
    out->n_state_blocks = static_cast<int32_t>(state->shape[0]);
    out->block_table = static_cast<const int32_t*>(bt->data);
    out->bt_stride = bt->stride[0];
    out->bt_rows = static_cast<int32_t>(bt->shape[0]);
    out->bt_cols = static_cast<int32_t>(bt->shape[1]);
    out->token_to_req = static_cast<const int32_t*>(t2r->data);
    out->positions = static_cast<const int32_t*>(pos->data);
    out->slot_mapping = static_cast<const int32_t*>(slot->data);
    out->num_tokens = static_cast<int32_t>(T);
    out->rms_w = static_cast<const float*>(w->data);
    out->eps = eps;
    out->cos_sin = static_cast<const float*>(cs->data);
    out->cs_stride = cs->stride[0];
    out->cs_rows = static_cast<int32_t>(cs->shape[0]);
    out->k_cache = static_cast<uint8_t*>(kc->data);
    out->kc_stride0 = kc->stride[0];
    out->kv_bs = static_cast<int32_t>(kc->shape[1]);
    out->n_kv_slots = kc->shape[0] * kc->shape[1];
    out->kv_slot_mapping = static_cast<const int32_t*>(kvs->data);
    out->compressed_out = nullptr;
  }
  if (state_bs) *state_bs = static_cast<int32_t>(sbs);
  g_last_error.clear();
  return DSV4_OK;
}

int run(const dsv4::C128Params& p, void* stream) {
  hipError_t err = dsv4::launch_c128_compress_store(p, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(DSV4_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(err));
  return DSV4_OK;
}

}  // namespace

extern "C" {

int dsv4_c128_validate(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                       const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                       const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                       const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                       const dsv4_tensor* kv_slot_mapping) {
  return validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, eps,
                      cos_sin, k_cache, kv_slot_mapping, nullptr);
}

int dsv4_c128_compress_store(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                             const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                             const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                             const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                             const dsv4_tensor* kv_slot_mapping, void* stream) {
  dsv4::C128Params p;
  int rc = validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                        eps, cos_sin, k_cache, kv_slot_mapping, &p);
  if (rc) return rc;
  if (p.num_tokens == 0) return DSV4_OK;
  return run(p, stream);
}

int dsv4_c128_compress_store_debug(const dsv4_tensor* state_cache,
                                   const dsv4_tensor* block_table,
                                   const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                   const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                   float eps, const dsv4_tensor* cos_sin,
                                   const dsv4_tensor* k_cache,
                                   const dsv4_tensor* kv_slot_mapping, float* compressed_out,
                                   void* stream) {
  dsv4::C128Params p;
  int rc = validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                        eps, cos_sin, k_cache, kv_slot_mapping, &p);
  if (rc) return rc;
  if (p.num_tokens == 0) return DSV4_OK;
  if (!compressed_out) return fail(DSV4_ERR_NULL, "compressed_out is NULL");
  if (!aligned16(compressed_out))
    return fail(DSV4_ERR_ALIGN, "compressed_out must be 16-byte aligned");
  p.compressed_out = compressed_out;
  return run(p, stream);
}

size_t dsv4_c128_workspace_bytes(int64_t num_tokens, int splits) {
  if (num_tokens <= 0) return 0;
  if (splits == 0) splits = dsv4::fanout_auto_splits(num_tokens);
  if (splits != 1 && splits != 2 && splits != 4 && splits != 8 && splits != 16) return 0;
  return dsv4::fanout_workspace_bytes(num_tokens, splits);
}

int dsv4_c128_compress_store_ex(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                                const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                float eps, const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                                const dsv4_tensor* kv_slot_mapping, float* compressed_out,
                                void* workspace, size_t workspace_bytes, int splits,
                                void* stream) {
  dsv4::C128Params p;
  int rc = validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                        eps, cos_sin, k_cache, kv_slot_mapping, &p);
  if (rc) return rc;
  if (splits != 0 && splits != 1 && splits != 2 && splits != 4 && splits != 8 && splits != 16)
    return fail(DSV4_ERR_ARG, "splits must be 0 (automatic), 1, 2, 4, 8 or 16 (got %d)", splits);
  if (compressed_out && !aligned16(compressed_out))
    return fail(DSV4_ERR_ALIGN, "compressed_out must be 16-byte aligned");
  if (p.num_tokens == 0) return DSV4_OK;
  if (splits > 1 && p.num_tokens > dsv4::kFanoutMaxTokens)
    return fail(DSV4_ERR_ARG, "the fan-out takes at most %lld tokens (got %d with %d splits)",
                static_cast<long long>(dsv4::kFanoutMaxTokens), p.num_tokens, splits);
  int s = splits;
  if (s == 0) {
    s = dsv4::fanout_auto_splits(p.num_tokens);
    if (s > 1 && (!workspace || workspace_bytes < dsv4::fanout_workspace_bytes(p.num_tokens, s)))
      s = 1;  // automatic mode never fails for want of a workspace: single pass
  }
  if (s > 1) {
    const size_t need = dsv4::fanout_workspace_bytes(p.num_tokens, s);
    if (!workspace || workspace_bytes < need)
      return fail(DSV4_ERR_ARG, "workspace of %zu bytes is too small: %d splits need %zu",
                  workspace_bytes, s, need);
    if (!aligned16(workspace)) return fail(DSV4_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  p.compressed_out = compressed_out;
  hipError_t err = dsv4::launch_c128_fanout(p, workspace, s,
                                            static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(DSV4_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(err));
  return DSV4_OK;
}

size_t dsv4_c128_varlen_workspace_bytes(int64_t num_tokens) {
  return dsv4::compacted_workspace_bytes(num_tokens);
}

int dsv4_c128_compress_store_varlen(const dsv4_tensor* state_cache,
                                    const dsv4_tensor* block_table,
                                    const dsv4_tensor* token_to_req,
                                    const dsv4_tensor* positions,
                                    const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                    float eps, const dsv4_tensor* cos_sin,
                                    const dsv4_tensor* k_cache,
                                    const dsv4_tensor* kv_slot_mapping, float* compressed_out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  dsv4::C128Params p;
  int rc = validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                        eps, cos_sin, k_cache, kv_slot_mapping, &p);
  if (rc) return rc;
  if (compressed_out && !aligned16(compressed_out))
    return fail(DSV4_ERR_ALIGN, "compressed_out must be 16-byte aligned");
  if (p.num_tokens == 0) return DSV4_OK;
  const size_t need = dsv4::compacted_workspace_bytes(p.num_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(DSV4_ERR_ARG, "workspace of %zu bytes is too small: %d tokens need %zu",
                workspace_bytes, p.num_tokens, need);
  if (!aligned16(workspace)) return fail(DSV4_ERR_ALIGN, "workspace must be 16-byte aligned");
  p.compressed_out = compressed_out;
  hipError_t err =
      dsv4::launch_c128_compacted(p, workspace, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(DSV4_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(err));
  return DSV4_OK;
}

int dsv4_c128_compress_store_varlen_noalloc(
    const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
    const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
    const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
    const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache, const dsv4_tensor* kv_slot_mapping,
    float* compressed_out, void* stream) {
  static_assert(dsv4::kStaticCompactedMaxTokens == DSV4_VARLEN_NOALLOC_MAX_TOKENS,
                "the header states the library's limit");
  dsv4::C128Params p;
  int rc = validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                        eps, cos_sin, k_cache, kv_slot_mapping, &p);
  if (rc) return rc;
  if (compressed_out && !aligned16(compressed_out))
    return fail(DSV4_ERR_ALIGN, "compressed_out must be 16-byte aligned");
  if (p.num_tokens == 0) return DSV4_OK;
  if (p.num_tokens > dsv4::kStaticCompactedMaxTokens)
    return fail(DSV4_ERR_ARG,
                "the allocation-free compacted schedule takes at most %lld tokens (got %d); "
                "use dsv4_c128_compress_store_varlen with a workspace",
                static_cast<long long>(dsv4::kStaticCompactedMaxTokens), p.num_tokens);
  p.compressed_out = compressed_out;
  hipError_t err = dsv4::launch_c128_compacted_static(p, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(DSV4_ERR_LAUNCH, "scratch lookup or kernel launch failed: %s",
                hipGetErrorString(err));
  return DSV4_OK;
}

int dsv4_c4_validate(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                     const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                     const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                     const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                     const dsv4_tensor* kv_slot_mapping) {
  return validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, eps,
                      cos_sin, k_cache, kv_slot_mapping, nullptr, kC4Layout);
}

int dsv4_c4_compress_store_debug(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                                 const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                 const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                 float eps, const dsv4_tensor* cos_sin,
                                 const dsv4_tensor* k_cache, const dsv4_tensor* kv_slot_mapping,
                                 float* compressed_out, void* stream) {
  dsv4::C128Params p;
  int32_t sbs = 0;
  int rc = validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                        eps, cos_sin, k_cache, kv_slot_mapping, &p, kC4Layout, &sbs);
  if (rc) return rc;
  if (compressed_out && !aligned16(compressed_out))
    return fail(DSV4_ERR_ALIGN, "compressed_out must be 16-byte aligned");
  if (p.num_tokens == 0) return DSV4_OK;
  p.compressed_out = compressed_out;
  hipError_t err = dsv4::launch_c4_compress_store(p, sbs, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(DSV4_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(err));
  return DSV4_OK;
}

int dsv4_c4_compress_store(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                           const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                           const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                           const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                           const dsv4_tensor* kv_slot_mapping, void* stream) {
  return dsv4_c4_compress_store_debug(state_cache, block_table, token_to_req, positions,
                                      slot_mapping, rms_w, eps, cos_sin, k_cache,
                                      kv_slot_mapping, nullptr, stream);
}

int dsv4_indexer_validate(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                          const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                          const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                          const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                          const dsv4_tensor* kv_slot_mapping) {
  return validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, eps,
                      cos_sin, k_cache, kv_slot_mapping, nullptr, kIndexerLayout);
}

int dsv4_indexer_compress_store_debug(const dsv4_tensor* state_cache,
                                      const dsv4_tensor* block_table,
                                      const dsv4_tensor* token_to_req,
                                      const dsv4_tensor* positions,
                                      const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                      float eps, const dsv4_tensor* cos_sin,
                                      const dsv4_tensor* k_cache,
                                      const dsv4_tensor* kv_slot_mapping, float* compressed_out,
                                      void* stream) {
  dsv4::C128Params p;
  int32_t sbs = 0;
  int rc = validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                        eps, cos_sin, k_cache, kv_slot_mapping, &p, kIndexerLayout, &sbs);
  if (rc) return rc;
  if (compressed_out && !aligned16(compressed_out))
    return fail(DSV4_ERR_ALIGN, "compressed_out must be 16-byte aligned");
  if (p.num_tokens == 0) return DSV4_OK;
  p.compressed_out = compressed_out;
  hipError_t err = dsv4::launch_indexer_compress_store(p, sbs, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(DSV4_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(err));
  return DSV4_OK;
}

int dsv4_indexer_compress_store(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                                const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                float eps, const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                                const dsv4_tensor* kv_slot_mapping, void* stream) {
  return dsv4_indexer_compress_store_debug(state_cache, block_table, token_to_req, positions,
                                           slot_mapping, rms_w, eps, cos_sin, k_cache,
                                           kv_slot_mapping, nullptr, stream);
}

int dsv4_indexer_mxfp4_validate(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                                const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                float eps, const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                                const dsv4_tensor* kv_slot_mapping) {
  return validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w, eps,
                      cos_sin, k_cache, kv_slot_mapping, nullptr, kIndexerMxfp4Layout);
}

int dsv4_indexer_mxfp4_compress_store_debug(
    const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
    const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
    const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
    const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache, const dsv4_tensor* kv_slot_mapping,
    float* compressed_out, void* stream) {
  dsv4::C128Params p;
  int32_t sbs = 0;
  int rc = validate_all(state_cache, block_table, token_to_req, positions, slot_mapping, rms_w,
                        eps, cos_sin, k_cache, kv_slot_mapping, &p, kIndexerMxfp4Layout, &sbs);
  if (rc) return rc;
  if (compressed_out && !aligned16(compressed_out))
    return fail(DSV4_ERR_ALIGN, "compressed_out must be 16-byte aligned");
  if (p.num_tokens == 0) return DSV4_OK;
  p.compressed_out = compressed_out;
  hipError_t err =
      dsv4::launch_indexer_mxfp4_compress_store(p, sbs, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(DSV4_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(err));
  return DSV4_OK;
}

int dsv4_indexer_mxfp4_compress_store(
    const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
    const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
    const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
    const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache, const dsv4_tensor* kv_slot_mapping,
    void* stream) {
  return dsv4_indexer_mxfp4_compress_store_debug(state_cache, block_table, token_to_req,
                                                 positions, slot_mapping, rms_w, eps, cos_sin,
                                                 k_cache, kv_slot_mapping, nullptr, stream);
}

int dsv4_e2m1_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n < 0) return fail(DSV4_ERR_SHAPE, "n must be >= 0");
  if (n == 0) return DSV4_OK;
  if (!in || !out) return fail(DSV4_ERR_NULL, "in/out is NULL");
  hipError_t err = dsv4::launch_e2m1_encode(in, out, n, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(DSV4_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(err));
  g_last_error.clear();
  return DSV4_OK;
}

int dsv4_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n < 0) return fail(DSV4_ERR_SHAPE, "n must be >= 0");
  if (n == 0) return DSV4_OK;
  if (!in || !out) return fail(DSV4_ERR_NULL, "in/out is NULL");
  hipError_t err = dsv4::launch_e4m3_encode(in, out, n, static_cast<hipStream_t>(stream));
  if (err != hipSuccess)
    return fail(DSV4_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(err));
  g_last_error.clear();
  return DSV4_OK;
}

const char* dsv4_last_error(void) { return g_last_error.c_str(); }

int dsv4_abi_version(void) { return DSV4_ABI_VERSION; }

}  // extern "C"
