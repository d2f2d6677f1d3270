/*
 * dsv4_c128.h -- C ABI of the DeepSeek-V4 sparse-attention compress-store path on
 * MI355X (gfx950): the C128 compressor (below), the C4 compressor (dsv4_c4_*) and the
 * indexer's compressor with its FP8 and MXFP4 caches (dsv4_indexer_*).
 *
 * What it computes (vLLM API page "fused_compress_quant_cache", DeepSeek-V4
 * common ops: the sparse-attention fused kernel
 * `_fused_kv_compress_norm_rope_insert_sparse_attn` and its launcher
 * `compress_norm_rope_store_triton`; vLLM PR 44230 "optimize the compressor
 * 128 split cutedsl kernel", sections Summary and Changes, for the C128 layout
 * limits and the wrapper-side validation):
 *
 *   For every token t whose state slot is >= 0 and whose position closes a
 *   128-row window ((pos+1) % 128 == 0):
 *     1. gather the window's 128 state rows q = pos-127 .. pos, row q at
 *        state_cache[block_table[token_to_req[t]][q / 8]][q % 8];
 *        a row is kv[0:512] followed by score[512:1024] (fp32);
 *     2. compressed[j] = sum_i softmax_i(score[i][j]) * kv[i][j], j < 512;
 *     3. RMSNorm: n = compressed / sqrt(mean(compressed^2) + eps) * rms_w;
 *     4. dims 0..447: round n to bf16, split into 7 blocks of 64, block
 *        exponent e = ceil(log2(max(absmax, 1e-4) / 448)), codes =
 *        E4M3FN(n * 2^-e) (OCP FP8, max 448), scale byte e + 127;
 *     5. dims 448..511: rotate interleaved pairs (448+2m, 449+2m), m < 32, by
 *        cos_sin[(pos / 128) * 128][m] (cos) and [32 + m] (sin); store bf16;
 *     6. if kv_slot_mapping[t] >= 0: with bs = k_cache.shape[1],
 *        blk = slot / bs, off = slot % bs, write the 576-byte record
 *        (448 codes, then 64 little-endian bf16) at byte
 *        blk*k_cache.stride[0] + off*576 and the 8 scale bytes (7 exponent
 *        bytes, then a zero pad byte) at blk*k_cache.stride[0] + bs*576 + off*8.
 *   Every other byte of k_cache stays unchanged.
 *
 * Tensor views.  Each argument is a dsv4_tensor: a caller-owned pointer, a
 * dtype code, a rank and shape/stride arrays.  Strides are in ELEMENTS; the
 * stride of every dimension longer than 1 is non-negative, and a tensor
 * spans at most 2^48 bytes from its first to its last element.
 * For the compute entry points every `data` pointer is device memory of the
 * current HIP device; the library never allocates, frees or keeps a pointer
 * after the call returns.  k_cache is written in place; every other tensor
 * is only read.
 *
 *   state_cache     f32 [S, 8, 1024]   stride[2] == 1, stride[1] >= 1024,
 *                                      stride[0] >= 8 * stride[1]; data and
 *                                      both strides 16-byte aligned
 *   block_table     i32 [R, M]         stride[1] == 1, M >= 16
 *   token_to_req    i32 [T]            contiguous
 *   positions       i32 [T]            contiguous; T <= DSV4_MAX_TOKENS
 *   slot_mapping    i32 [T]            contiguous; only its sign is used
 *   rms_w           f32 [512]          contiguous, 16-byte aligned
 *   cos_sin         f32 [P, >= 64]     stride[1] == 1; cos in [0,32), sin in [32,64)
 *   k_cache         u8  [B, bs, 584]   stride[2] == 1, stride[1] == 584,
 *                                      stride[0] >= bs*584 and a multiple of
 *                                      8; data 8-byte aligned.  Only bs and
 *                                      stride[0] give the layout: the view is a
 *                                      byte container for the block format above
 *   kv_slot_mapping i32 [T]            contiguous
 *
 * Calls are stream-ordered and asynchronous: no host synchronisation and no
 * device-to-host reads.  T == 0 is a valid no-op.  Calls keep no device state
 * of the library's own between calls (except dsv4_c128_compress_store_varlen_noalloc,
 * below), so calls on different streams may overlap when they share no output
 * and no workspace.
 *
 * Errors.  Entry points return DSV4_OK (0) or a negative DSV4_ERR_* code.  On
 * any validation error nothing is launched and k_cache is untouched;
 * dsv4_last_error() then holds a message (per calling thread).
 *
 * Values that live in device memory are not validated by the host (that
 * would need a synchronisation): block ids, request ids, window columns,
 * RoPE rows and kv slots.  The kernel range-checks each of them and a token
 * with any out-of-range index writes nothing.  Two active tokens with the
 * same kv slot race (the pages leave this undefined too).
 */
#ifndef DSV4_C128_H
#define DSV4_C128_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSV4_ABI_VERSION 8

/* Most tokens one call takes (2^27).  The largest launch grid, the staged schedule's 16
   work-items per token, then stays within half of the 32-bit work-item count of a dispatch.
   Longer batches are split by the caller: tokens are independent. */
#define DSV4_MAX_TOKENS 134217728

enum dsv4_dtype { DSV4_F32 = 1, DSV4_I32 = 2, DSV4_U8 = 3 };

enum dsv4_status {
  DSV4_OK = 0,
  DSV4_ERR_NULL = -1,   /* a required pointer is NULL */
  DSV4_ERR_DTYPE = -2,  /* wrong dtype code */
  DSV4_ERR_RANK = -3,   /* wrong number of dimensions */
  DSV4_ERR_SHAPE = -4,  /* state block != 8, state row != 1024 (head 512 + score 512),
                           k_cache row != 584, rms_w != 512, cos_sin < 64 columns,
                           block table < 16 columns, token arrays of different length,
                           more than DSV4_MAX_TOKENS tokens, or a size above INT32_MAX */
  DSV4_ERR_STRIDE = -5, /* inner stride != 1, overlapping rows/blocks, k_cache stride[0]
                           below bs*584, a negative stride, or a span above 2^48 bytes */
  DSV4_ERR_ALIGN = -6,  /* a pointer or stride breaks the alignment stated above */
  DSV4_ERR_LAUNCH = -7, /* the HIP runtime reported an error at launch */
  DSV4_ERR_ARG = -8     /* an argument outside its documented set (splits, workspace size) */
};

typedef struct dsv4_tensor {
  void* data;        /* first element */
  int32_t dtype;     /* enum dsv4_dtype */
  int32_t ndim;      /* 1..4 */
  int64_t shape[4];
  int64_t stride[4]; /* in elements */
} dsv4_tensor;

/*
 * The fused compress-store (steps 1-6 above) for all T tokens, launched on
 * `stream` (a hipStream_t; NULL means the default stream).
 * `eps` is the RMSNorm epsilon.
 *
 * Below 2048 tokens one workgroup handles each token (the single pass).  From
 * 2048 tokens on, one workgroup per compute unit tests the gate of every token,
 * ranks the tokens that pass, and takes an equal share of them, so a batch in
 * which few tokens close a window (chunked prefill) spreads as evenly as one in
 * which all do; it streams its share in stages of up to 64 tokens and inserts a
 * stage's records after the stage's last state read, which keeps the k_cache
 * writes out of the state stream (the staged schedule).  It merges 8 partial
 * row groups per token instead of 4, so a code can differ from the single
 * pass's by one step of fp32 rounding; both agree with the definition to the
 * same tolerance.  No scratch memory, one kernel launch.
 */
int dsv4_c128_compress_store(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                             const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                             const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                             const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                             const dsv4_tensor* kv_slot_mapping, void* stream);

/*
 * Same as dsv4_c128_compress_store, and also stores the fp32 `compressed`
 * vector (step 2) of each token that passes the gate to
 * compressed_out[t * 512 + j] (device memory, [T, 512] row-major, 16-byte
 * aligned).  Rows of tokens that do not pass the gate are left unchanged.
 * For tests; the k_cache bytes are identical to the plain entry point's.
 */
int dsv4_c128_compress_store_debug(const dsv4_tensor* state_cache,
                                   const dsv4_tensor* block_table,
                                   const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                   const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                   float eps, const dsv4_tensor* cos_sin,
                                   const dsv4_tensor* k_cache,
                                   const dsv4_tensor* kv_slot_mapping, float* compressed_out,
                                   void* stream);

/*
 * Small-batch fan-out.  The same computation as dsv4_c128_compress_store, with each token's 16
 * window blocks split over `splits` workgroups (grid T x splits) that write partial softmax
 * states to `workspace`; the last workgroup of a token to finish (found with a per-token arrival
 * counter in the workspace) merges them and runs the epilogue, in the same kernel.  It exists
 * because one workgroup per token leaves most of the 256 CUs idle when T is small (decode
 * batches of up to about a hundred tokens); the pages' own split kernel (vLLM
 * fused_compress_quant_cache page, `_compress_gather_split_sparse_attn` and
 * `_pick_compress_num_splits`) has the same purpose.
 *
 *   splits          0 = the library's choice for T (see dsv4_c128_workspace_bytes), or 1, 2,
 *                   4, 8, 16.  1 is the single-pass kernel.  With splits > 1, T may be at most
 *                   4096 (else DSV4_ERR_ARG; with splits == 0 the library never splits there).
 *   workspace       device memory of at least dsv4_c128_workspace_bytes(T, splits) bytes,
 *                   16-byte aligned, owned by the caller.  Its first 16384 bytes hold the
 *                   arrival counters: they must be zero before the first call that splits (fill
 *                   the buffer with zeros once, when it is allocated), and every call leaves them
 *                   zero again, so the same workspace serves any number of later calls with any
 *                   T and splits.  The rest is scratch.  Calls that share a workspace must be
 *                   ordered on one stream.  With splits == 0 and no (or too small a) workspace
 *                   the single pass runs; with explicit splits > 1 it is DSV4_ERR_ARG.
 *   compressed_out  NULL, or as in dsv4_c128_compress_store_debug.
 *
 * k_cache results equal the single pass's up to the fp32 summation order of the pooling, and do
 * not depend on which workgroup of a token finishes last (the partials are merged in split
 * order).
 */
int dsv4_c128_compress_store_ex(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                                const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                float eps, const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                                const dsv4_tensor* kv_slot_mapping, float* compressed_out,
                                void* workspace, size_t workspace_bytes, int splits, void* stream);

/*
 * Bytes of workspace dsv4_c128_compress_store_ex needs for num_tokens tokens and `splits`
 * (0 = the library's choice: 8 for num_tokens <= 16, 4 for 17..64, 2 for 65..128, 1 above):
 * 16384 + num_tokens * splits * 6144.  0 when no workspace is needed (splits 1) or the
 * combination is not valid (splits not in {0, 1, 2, 4, 8, 16}, or more than 4096 tokens with
 * splits > 1).  Host-only; no HIP call.
 */
size_t dsv4_c128_workspace_bytes(int64_t num_tokens, int splits);

/*
 * Compacted schedule for long varlen batches (chunked prefill).  The same computation as
 * dsv4_c128_compress_store.  Only tokens whose position closes a 128-row window do any work
 * (vLLM fused_compress_quant_cache page, sparse-attention kernel: one program per token that
 * returns early unless (pos + 1) % 128 == 0), and in a prefill batch that is about one token in
 * 128.  A first kernel tests the gate on every token and writes the passing token indices,
 * compacted, to `workspace`; a persistent grid of workgroups then processes only those tokens.
 * Per token it computes exactly what the single pass computes, so below 2048 tokens its results
 * equal dsv4_c128_compress_store's bit for bit; they never depend on the schedule.  For decode
 * batches, where every token passes, the plain entry point is faster.
 *
 *   workspace       device memory of at least dsv4_c128_varlen_workspace_bytes(T) bytes,
 *                   16-byte aligned, owned by the caller; no initialisation needed, scratch after
 *                   the call.  Calls that share a workspace must be ordered on one stream.
 *                   NULL or too small: DSV4_ERR_ARG (unless T == 0).
 *   compressed_out  NULL, or as in dsv4_c128_compress_store_debug.
 */
int dsv4_c128_compress_store_varlen(const dsv4_tensor* state_cache,
                                    const dsv4_tensor* block_table,
                                    const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                    const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                    float eps, const dsv4_tensor* cos_sin,
                                    const dsv4_tensor* k_cache,
                                    const dsv4_tensor* kv_slot_mapping, float* compressed_out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace dsv4_c128_compress_store_varlen needs for num_tokens tokens: 4 * (1024 +
 * num_tokens) rounded up to a multiple of 16 (per-scan-block counts, then the compacted token
 * list); 0 for num_tokens <= 0.  Host-only; no HIP call.
 */
size_t dsv4_c128_varlen_workspace_bytes(int64_t num_tokens);

/* Most tokens dsv4_c128_compress_store_varlen_noalloc takes in one call (2^20). */
#define DSV4_VARLEN_NOALLOC_MAX_TOKENS 1048576

/*
 * dsv4_c128_compress_store_varlen without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * The same two kernels and the same results, bit for bit; the scan counts and the compacted
 * token list live in a fixed array inside the library instead: 4 * (1024 + 2^20) bytes
 * (4 MiB + 4 KiB) of device memory on each device the library runs on, held until the process
 * ends.  The call allocates and frees nothing.
 *
 *   T               at most DSV4_VARLEN_NOALLOC_MAX_TOKENS, else DSV4_ERR_ARG before any HIP
 *                   call (split longer batches: tokens are independent).
 *   compressed_out  NULL, or as in dsv4_c128_compress_store_debug.
 *
 * The array needs no initialisation: each call's scan writes every count and list entry that
 * the same call reads.  All calls on one device share the array, so calls that overlap in time
 * on one device race (two streams, or two host threads); order them on one stream.  The first
 * call on a device looks up the array's device address (hipGetSymbolAddress) with that device
 * current; make it outside graph capture.  An error of that lookup is DSV4_ERR_LAUNCH.
 */
int dsv4_c128_compress_store_varlen_noalloc(
    const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
    const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
    const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
    const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache, const dsv4_tensor* kv_slot_mapping,
    float* compressed_out, void* stream);

/*
 * The C4 compressor: the same fused computation with compress ratio 4 and an overlapping
 * window (vLLM fused_compress_quant_cache page, sparse-attention fused kernel, with
 * COMPRESS_RATIO = 4 and OVERLAP = 1; vLLM PR 44230, Summary: C4 keeps its fused path).
 * For every token t whose state slot is >= 0 and whose position closes a 4-row window
 * ((pos+1) % 4 == 0):
 *   1. the window is the 8 rows q = pos-7 .. pos (rows with q < 0, which exist only at
 *      pos = 3, take no part), row q at state_cache[block_table[token_to_req[t]][q / bs]]
 *      [q % bs] with bs = state_cache.shape[1];
 *   2. a state row is kv[0:1024] | score[1024:2048]; window row i < 4 (the previous window)
 *      contributes kv[j] and score[1024 + j], row i >= 4 (the current window) kv[512 + j] and
 *      score[1536 + j], for output column j < 512;
 *   3. compressed[j] = sum_i softmax_i(score) * kv over those rows, then steps 3-6 of the C128
 *      path with the RoPE table row (pos / 4) * 4, into the same 584-byte k_cache layout.
 *
 *   state_cache     f32 [S, bs, 2048]  bs >= 1 (any block size), stride[2] == 1,
 *                                      stride[1] >= 2048, stride[0] >= bs * stride[1]; data
 *                                      and both strides 16-byte aligned
 *   block_table     i32 [R, M]         stride[1] == 1, M >= 1 (a token needs column pos / bs)
 *   every other argument as for dsv4_c128_compress_store.
 * Device-resident indices are range-checked as in the C128 path.
 */
int dsv4_c4_compress_store(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                           const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                           const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                           const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                           const dsv4_tensor* kv_slot_mapping, void* stream);

/* dsv4_c4_compress_store that also writes the fp32 pooled vectors, as
 * dsv4_c128_compress_store_debug does (compressed_out may be NULL). */
int dsv4_c4_compress_store_debug(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                                 const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                 const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                 float eps, const dsv4_tensor* cos_sin,
                                 const dsv4_tensor* k_cache, const dsv4_tensor* kv_slot_mapping,
                                 float* compressed_out, void* stream);

/* Host-only validation of the C4 descriptors (as dsv4_c128_validate). */
int dsv4_c4_validate(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                     const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                     const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                     const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                     const dsv4_tensor* kv_slot_mapping);

/*
 * The indexer's FP8 compressor (vLLM fused_compress_quant_cache page, kernel
 * `_fused_kv_compress_norm_rope_insert_indexer_attn`), on the overlapping window of compress
 * ratio 4.  For every token t whose state slot is >= 0 and (pos+1) % 4 == 0:
 *   1. window rows q = pos-7 .. pos as for dsv4_c4_compress_store (rows with q < 0 left out),
 *      with head 128: a state row is kv[0:256] | score[256:512]; window row i < 4 contributes
 *      kv[j] and score[256 + j], row i >= 4 kv[128 + j] and score[384 + j], j < 128;
 *   2. compressed[j] = sum_i softmax_i(score) * kv, j < 128; RMSNorm over 128 with rms_w[128];
 *   3. RoPE first: dims 64..127 as interleaved pairs (64+2m, 65+2m), m < 32, rotated by
 *      cos_sin[(pos / 4) * 4][m] and [32 + m]; dims 0..63 unchanged;
 *   4. then one quantisation block over all 128 dims: bf16 round trip, absmax (floor 1e-4),
 *      e = ceil(log2(absmax / 448)), codes = E4M3FN(x * 2^-e), scale = 2^e as fp32;
 *   5. if kv_slot_mapping[t] >= 0: with bs = k_cache.shape[1], blk = slot / bs, off = slot %
 *      bs, the 128 codes at byte blk*k_cache.stride[0] + off*128 and the fp32 scale
 *      (little-endian) at blk*k_cache.stride[0] + bs*128 + off*4.
 *
 *   state_cache     f32 [S, bs, 512]   bs >= 1, strides and alignment as for C4 (stride[1] >= 512)
 *   rms_w           f32 [128]          contiguous, 16-byte aligned
 *   k_cache         u8  [B, bs, 132]   stride[2] == 1, stride[1] == 132, stride[0] >= bs*132
 *                                      and a multiple of 4; data 4-byte aligned
 *   every other argument as for dsv4_c4_compress_store; compressed_out of the debug entry
 *   point is [T, 128] fp32.
 */
int dsv4_indexer_compress_store(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                                const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                float eps, const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                                const dsv4_tensor* kv_slot_mapping, void* stream);

/* dsv4_indexer_compress_store that also writes the fp32 pooled vectors ([T, 128], 16-byte
 * aligned; rows of tokens that do not pass the gate are left unchanged; may be NULL). */
int dsv4_indexer_compress_store_debug(const dsv4_tensor* state_cache,
                                      const dsv4_tensor* block_table,
                                      const dsv4_tensor* token_to_req,
                                      const dsv4_tensor* positions,
                                      const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                      float eps, const dsv4_tensor* cos_sin,
                                      const dsv4_tensor* k_cache,
                                      const dsv4_tensor* kv_slot_mapping, float* compressed_out,
                                      void* stream);

/* Host-only validation of indexer descriptors (as dsv4_c128_validate). */
int dsv4_indexer_validate(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                          const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                          const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                          const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                          const dsv4_tensor* kv_slot_mapping);

/*
 * The indexer's compressor with the MXFP4 cache (vLLM fused_compress_quant_cache page, kernel
 * `_fused_kv_compress_norm_rope_insert_indexer_mxfp4_attn` and its MXFP4-format notes).  Steps
 * 1-3 are those of dsv4_indexer_compress_store; then:
 *   4. every rotated value (held in fp32; dims 0..63 unrotated) is rounded to bf16;
 *   5. four blocks of 32 consecutive dims: absmax (floor 6 * 2^-126), e = ceil(log2(absmax *
 *      fl32(1/6))) computed on the fp32 product, clamped to [-127, 127]; codes = E2M1(x * 2^-e),
 *      rounded to nearest with ties to the even code, sign kept, saturating at 6 (the page
 *      does not print its conversion; this is the OCP E2M1 format's round to nearest even);
 *   6. if kv_slot_mapping[t] >= 0: with bs = k_cache.shape[1], blk = slot / bs, off = slot %
 *      bs, 64 bytes at blk*k_cache.stride[0] + off*64, byte p holding dim 2p in its low
 *      nibble and dim 2p+1 in its high nibble, and the 4 scale bytes e + 127 (one per block)
 *      at blk*k_cache.stride[0] + bs*64 + off*4.
 *
 *   k_cache         u8  [B, bs, 68]    stride[2] == 1, stride[1] == 68, stride[0] >= bs*68 and
 *                                      a multiple of 4; data 4-byte aligned
 *   every other argument, the gate, the range checks and the errors as for
 *   dsv4_indexer_compress_store; compressed_out of the debug entry point is [T, 128] fp32.
 */
int dsv4_indexer_mxfp4_compress_store(
    const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
    const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
    const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
    const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache, const dsv4_tensor* kv_slot_mapping,
    void* stream);

/* dsv4_indexer_mxfp4_compress_store that also writes the fp32 pooled vectors ([T, 128],
 * 16-byte aligned; rows of tokens that do not pass the gate are left unchanged; may be NULL). */
int dsv4_indexer_mxfp4_compress_store_debug(
    const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
    const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
    const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
    const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache, const dsv4_tensor* kv_slot_mapping,
    float* compressed_out, void* stream);

/* Host-only validation of MXFP4 indexer descriptors (as dsv4_c128_validate). */
int dsv4_indexer_mxfp4_validate(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                                const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                                const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w,
                                float eps, const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                                const dsv4_tensor* kv_slot_mapping);

/*
 * Host-only validation of the descriptors, exactly as the compute entry
 * points do it.  Makes no HIP call and dereferences no `data` pointer, so it
 * runs without a GPU.  Returns DSV4_OK or the DSV4_ERR_* the compute entry
 * point would return.
 */
int dsv4_c128_validate(const dsv4_tensor* state_cache, const dsv4_tensor* block_table,
                       const dsv4_tensor* token_to_req, const dsv4_tensor* positions,
                       const dsv4_tensor* slot_mapping, const dsv4_tensor* rms_w, float eps,
                       const dsv4_tensor* cos_sin, const dsv4_tensor* k_cache,
                       const dsv4_tensor* kv_slot_mapping);

/*
 * The E4M3FN encoder of step 4 as the kernel runs it (clamp to [-448, 448],
 * then round to nearest even), applied to n fp32 values: out[i] =
 * code(in[i]).  Device pointers, no alignment needed beyond 4 bytes for
 * `in`.  For exhaustive tests of the hardware conversion (OCP FP8 E4M3FN on
 * gfx950).
 */
int dsv4_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream);

/*
 * The E2M1 encoder of the MXFP4 cache as the kernel runs it, applied to n fp32 values:
 * out[i] = code(in[i]) in the low nibble (bit 3 the sign), the high nibble 0.  Device pointers.
 * For exhaustive tests of the encoder.
 */
int dsv4_e2m1_encode(const float* in, uint8_t* out, int64_t n, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* dsv4_last_error(void);

/* DSV4_ABI_VERSION of the loaded library. */
int dsv4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSV4_C128_H */
