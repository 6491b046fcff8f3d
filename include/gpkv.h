/*
 * gpkv.h -- C ABI of the paged GQA decode-attention library for AMD MI355X (gfx950).
 *
 * Single-token decode attention over a paged KV cache, its write path and the
 * Quest long-context variant. The operations:
 *
 *   gpkv_reshape_and_cache           write new tokens' K/V rows into the cache
 *   gpkv_reshape_and_cache_quest     ... and update those blocks' Quest key min / max
 *   gpkv_paged_attention_decode      dense GQA paged attention (split-KV + combine)
 *   gpkv_paged_attention_decode_append   ... with the step's cache write (decode append)
 *   gpkv_paged_attention_decode_noalloc  ... without a workspace (fixed device array)
 *   gpkv_quest_block_metadata        per-block, per-channel key min / max
 *   gpkv_quest_select_topk           Quest block scores + Top-K per KV head
 *   gpkv_sparse_paged_attention_decode  exact attention over the selected blocks
 *   gpkv_quest_decode                selection and sparse attention in one call
 *   gpkv_quest_decode_append         ... with the step's cache write (decode append)
 *   ..._fp8 variants of the write and both attention calls over E4M3 caches,
 *   and gpkv_paged_attention_decode_fp8_append (the FP8 dense step in one call)
 *   gpkv_paged_attention_varlen      multi-token queries (causal, right-aligned)
 *
 * Sources, by page title and section:
 *   [ASC]  "Ascend Kernel-to-Serving Pipeline": sections "ReshapeAndCache",
 *          "GQA Paged Attention", "Quest Sparse Attention", "single-operator
 *          correctness", "Sparse precision", "memory optimisation".
 *   [TL18] TileLang tutorial, chapter 18 (end-to-end inference serving):
 *          2.4 KV-cache structure, 2.6 paged KV, 2.7 varlen batches, 3.3 varlen
 *          kernel requirements, 4.1 split-KV decode attention,
 *          2.5 item 3 and 3.1 item 4 (KV quantisation as the long-context lever),
 *          6.1 kernels on the framework's current stream, 6.2 graph capture,
 *          8 item (2) the per-step KV write.
 *   [DSA]  The article on adapting a sparse-attention model to a new accelerator:
 *          section on the four key levels of the sparse-attention kernel, items 2
 *          (per-block metadata, updated block by block at decode) and 3 (KV-cache
 *          update merged into the decode kernel's launch).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - bf16 tensors are passed as `const void*` / `void*` to raw bfloat16 bits.
 *    Every tensor is contiguous, row-major, in device memory (HBM), except where
 *    a comment says otherwise.
 *  - KV cache layout ([TL18] 2.6): key_cache and value_cache are each
 *    [num_blocks, block_size, num_kv_heads, head_dim] bf16. Token t of sequence b
 *    lives in physical block block_tables[b * max_blocks_per_seq + t / block_size],
 *    row t % block_size.
 *  - block_tables: [batch, max_blocks_per_seq] int32; entries at logical index
 *    >= ceil(context_lens[b] / block_size) are never read.
 *  - context_lens: [batch] int32, each in [0, max_context_len]. It includes the
 *    token written by this step's reshape_and_cache.
 *  - GQA ([ASC] "GQA Paged Attention"): num_q_heads is a multiple of
 *    num_kv_heads; query head h reads KV head h / (num_q_heads / num_kv_heads).
 *  - Supported shapes: head_dim in {64, 128}; block_size in {16, 32, 64, 128};
 *    group size num_q_heads / num_kv_heads in [1, 16].
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on it: no allocation, no host<->device copy, no
 *    synchronisation ([TL18] 6.1). Grids depend only on host scalars, so the
 *    calls can be captured into a HIP graph ([TL18] 6.2).
 *  - Ownership: the caller owns every buffer (caches, metadata, outputs and
 *    workspaces); the library keeps no pointer after a call returns.
 *  - Errors: arguments are checked on the host before any launch. A failing
 *    check returns a negative gpkv_status, launches nothing, and stores a
 *    message readable with gpkv_last_error_message() (per thread). A launch
 *    failure reported by the HIP runtime returns GPKV_ERR_HIP. Device-side
 *    contents (block ids, lengths, slots, selected ids) are preconditions and
 *    are not checked; kernels still skip out-of-range slots and selected ids.
 */
#ifndef GPKV_H_
#define GPKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPKV_OK = 0,
  GPKV_ERR_NULL = -1,        /* a required pointer is NULL                        */
  GPKV_ERR_SHAPE = -2,       /* inconsistent or negative sizes                    */
  GPKV_ERR_UNSUPPORTED = -3, /* head_dim / block_size / group size not supported  */
  GPKV_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required        */
  GPKV_ERR_HIP = -5          /* the HIP runtime reported an error at launch       */
} gpkv_status;

/* ReshapeAndCache ([ASC] "ReshapeAndCache").
 * For each new token i < num_tokens with s = slot_mapping[i]:
 *   s < 0                 -> the token is skipped;
 *   otherwise block = s / block_size, row = s % block_size, and
 *   key_cache[block, row, :, :] = key[i], value_cache[block, row, :, :] = value[i].
 * key, value: [num_tokens, num_kv_heads, head_dim] bf16 (read).
 * key_cache, value_cache: [num_blocks, block_size, num_kv_heads, head_dim] bf16,
 *   modified in place; rows not named by a slot are left untouched.
 * slot_mapping: [num_tokens] int64. Slots >= num_blocks * block_size are skipped
 *   (precondition violation, tolerated for memory safety); two tokens naming the
 *   same slot is a precondition violation with an unspecified winner.
 * num_tokens == 0 is a no-op. */
int gpkv_reshape_and_cache(const void* key, const void* value, void* key_cache,
                           void* value_cache, const int64_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, void* stream);

/* Fused write path: ReshapeAndCache plus the Quest metadata of the written blocks,
 * in one launch ([ASC] "ReshapeAndCache" and "Quest Sparse Attention"; the per-step
 * KV write is a real cost, [TL18] 8 item (2); the cache update shares a launch and
 * block metadata is updated incrementally at decode, [DSA] items 2-3). Writes key[i] / value[i] exactly as gpkv_reshape_and_cache and, for
 * each written token with block = slot / bs and row = slot % bs, sets for every KV
 * head g and channel c:
 *   row == 0:  key_min[block, g, c] = key_max[block, g, c] = key[i, g, c]
 *   row  > 0:  key_min[block, g, c] = min(key_min[block, g, c], key[i, g, c]), same for max.
 * This equals recomputing the block's metadata over rows 0..row (as
 * gpkv_quest_block_metadata with last_block_only does) when the token is the newest
 * valid row of its block and the block's metadata covered rows 0..row-1 before the
 * call -- the decode-append case. At most one token per block per call
 * (precondition). key_min, key_max: [num_blocks, num_kv_heads, head_dim] bf16. */
int gpkv_reshape_and_cache_quest(const void* key, const void* value, void* key_cache,
                                 void* value_cache, void* key_min, void* key_max,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int64_t num_blocks, void* stream);

/* Bytes of workspace gpkv_paged_attention_decode needs for these sizes (0 if the
 * sizes are invalid). The workspace holds split-KV partial outputs and their
 * log-sum-exp ([TL18] 4.1). */
size_t gpkv_paged_attention_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t max_context_len);

/* Dense GQA paged decode attention ([ASC] "GQA Paged Attention"; [TL18] 2.6, 4.1).
 * out[b, h, :] = sum_t p_t V_t with p = softmax_t(scale * q[b, h, :] . K_t) over the
 * tokens t < context_lens[b] of sequence b (ragged last block masked; a
 * sequence with context 0 gets a zero row). K_t, V_t are KV head h / G of the
 * token's cache row.
 * out: [batch, num_q_heads, head_dim] float32 (written).
 * query: [batch, num_q_heads, head_dim] bf16.
 * max_context_len: a host-side upper bound of context_lens (sizes the grid and
 *   the workspace); must be <= max_blocks_per_seq * block_size.
 * scale: the softmax scale (typically 1/sqrt(head_dim)).
 * workspace: device memory of at least gpkv_paged_attention_workspace_bytes(...)
 *   bytes; its contents on entry are ignored and on exit are unspecified. */
int gpkv_paged_attention_decode(float* out, const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, int32_t batch,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len,
                                float scale, void* workspace, size_t workspace_bytes,
                                void* stream);

/* The step's cache write merged into the dense decode call (the KV-cache update
 * sharing the decode kernel's launch, [DSA] items 2-3; the per-step KV write is a
 * real cost, [TL18] 8 item (2)): one call, two launches, for the decode-append case
 * where token b of key / value is sequence b's newest token, at position
 * context_lens[b] - 1. With s = slot_mapping[b]:
 *   0 <= s < num_blocks * block_size: key[b] / value[b] are written to slot s as
 *     gpkv_reshape_and_cache writes them and, when key_min / key_max are given,
 *     folded into that block's Quest metadata as gpkv_reshape_and_cache_quest does;
 *     the attention of sequence b takes its position context_lens[b] - 1 from
 *     key[b] / value[b] (when context_lens[b] >= 1);
 *   otherwise: nothing is written and the attention reads the cache as
 *     gpkv_paged_attention_decode does.
 * The result equals gpkv_reshape_and_cache(_quest) over the batch's tokens followed
 * by gpkv_paged_attention_decode (attention within the same tolerance, caches and
 * metadata bit for bit) under the precondition of the decode-append case: every
 * in-pool slot_mapping[b] is the slot of sequence b's position context_lens[b] - 1
 * (block_tables[b, (context_lens[b] - 1) / block_size], row
 * (context_lens[b] - 1) % block_size), and no other sequence reads that slot. The
 * split phase reads the cache up to position context_lens[b] - 2 of such a sequence;
 * the combine merges the new token as one more unit and writes it into the cache.
 * key, value: [batch, num_kv_heads, head_dim] bf16. slot_mapping: [batch] int64.
 * key_min, key_max: [num_blocks, num_kv_heads, head_dim] bf16, both null (no
 *   metadata) or both given. key_cache, value_cache (and the metadata) are modified
 *   in place at the written slots only.
 * Everything else (out, query, tables, sizes, scale, workspace of
 * gpkv_paged_attention_workspace_bytes, errors) as gpkv_paged_attention_decode;
 * one of key_min / key_max null without the other is GPKV_ERR_NULL. */
int gpkv_paged_attention_decode_append(float* out, const void* query, const void* key,
                                       const void* value, void* key_cache, void* value_cache,
                                       void* key_min, void* key_max,
                                       const int64_t* slot_mapping,
                                       const int32_t* block_tables,
                                       const int32_t* context_lens, int32_t batch,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       float scale, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* gpkv_paged_attention_decode without allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, result and errors as gpkv_paged_attention_decode,
 * minus the workspace: the split-KV partial rows live in a device array inside the
 * library, GPKV_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held from the first call on
 * that GPU until the process ends; its device address is looked up once per device
 * on the first call. The call allocates nothing (no hipMalloc, no library
 * allocation). Sizes whose workspace (gpkv_paged_attention_workspace_bytes) exceeds
 * the array return GPKV_ERR_WORKSPACE and launch nothing; a failed address lookup
 * returns GPKV_ERR_HIP. Every call on one GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (different streams, or threads) race and give
 * unspecified results: the caller serialises them. Nothing in the array has to start
 * at zero; its contents after a call are unspecified. */
#define GPKV_NOALLOC_SCRATCH_BYTES (32u << 20)
int gpkv_paged_attention_decode_noalloc(float* out, const void* query, const void* key_cache,
                                        const void* value_cache, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t batch,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                        int32_t max_blocks_per_seq, int32_t max_context_len,
                                        float scale, void* stream);

/* Quest block metadata ([ASC] "Quest Sparse Attention": blocks are scored at low
 * cost; tokens past the context are skipped). For every sequence b and logical
 * block lb < ceil(context_lens[b] / block_size) -- only the last one when
 * last_block_only != 0 -- with pb = block_tables[b, lb] and
 * n = min(block_size, context_lens[b] - lb * block_size) valid rows:
 *   key_min[pb, g, c] = min over rows t < n of key_cache[pb, t, g, c]
 *   key_max[pb, g, c] = max over rows t < n of key_cache[pb, t, g, c]
 * key_min, key_max: [num_blocks, num_kv_heads, head_dim] bf16, written only at
 *   referenced blocks (the rest keep their contents). Results are exact (they are
 *   input values). A physical block referenced by two sequences is a
 *   precondition violation. */
int gpkv_quest_block_metadata(void* key_min, void* key_max, const void* key_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t batch, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len,
                              int32_t last_block_only, void* stream);

/* Bytes of workspace gpkv_quest_select_topk needs (per-block scores in float64). */
size_t gpkv_quest_select_workspace_bytes(int32_t batch, int32_t num_kv_heads,
                                         int32_t max_blocks_per_seq);

/* Quest block scoring and Top-K selection ([ASC] "Quest Sparse Attention").
 * For each (b, KV head g) and each logical block lb < nb_b = ceil(ctx_b / bs):
 *   score(lb) = sum over the group's query heads h and channels c of
 *               max(q[b,h,c] * key_min[pb,g,c], q[b,h,c] * key_max[pb,g,c])
 * computed in float64 (bf16 products are exact; the sum is rounded in float64).
 * The min(topk_blocks, nb_b) highest-scoring blocks are kept (equal scores: the
 * lower logical index wins) and written in ascending order of logical index,
 * padded with -1 up to topk_blocks.
 * topk_indices: [batch, num_kv_heads, topk_blocks] int32 (written).
 * key_min, key_max: as produced by gpkv_quest_block_metadata.
 * topk_blocks >= 1. */
int gpkv_quest_select_topk(int32_t* topk_indices, const void* query, const void* key_min,
                           const void* key_max, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_context_len, int32_t topk_blocks, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Bytes of workspace gpkv_sparse_paged_attention_decode needs. */
size_t gpkv_sparse_attention_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t topk_blocks);

/* Quest sparse paged attention ([ASC] "Quest Sparse Attention", "Sparse precision").
 * Exact softmax attention of every query head of group g over only the tokens of
 * the logical blocks listed in topk_indices[b, g, :] (tokens >= context_lens[b]
 * masked). Entries equal to -1 (or outside [0, nb_b)) are ignored; listing a
 * block twice is a precondition violation. Output as in
 * gpkv_paged_attention_decode (zero row when no token is selected).
 * topk_indices: [batch, num_kv_heads, topk_blocks] int32 logical block ids.
 * When the batch's (sequence, KV head) pairs fill the GPU, each pair is one
 * workgroup that writes its rows directly (one launch, workspace untouched);
 * otherwise the split phase writes partial rows to the workspace and a second
 * launch combines them. The workspace size is the same either way. */
int gpkv_sparse_paged_attention_decode(float* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       const int32_t* context_lens,
                                       const int32_t* topk_indices, int32_t batch,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int64_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_context_len, int32_t topk_blocks,
                                       float scale, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Quest decode step in one call ([ASC] "Quest Sparse Attention"; "test results and
 * interpretation" item 4 names the sparse path's costs: scoring, Top-K, indexing
 * and the scheduling of several kernels): the result of gpkv_quest_select_topk followed by
 * gpkv_sparse_paged_attention_decode on the same arguments. topk_indices
 * [batch, num_kv_heads, topk_blocks] int32 receives the selection (ascending, -1
 * padding), out [batch, num_q_heads, head_dim] fp32 the attention over it. key_min /
 * key_max as for gpkv_quest_select_topk, caches and scale as for the attention
 * calls. When the (sequence, KV head) pairs fill between half of the GPU's CUs
 * and all of them, or each pair reads little (at most 256 KB of metadata and
 * selected K/V), one workgroup per pair selects in LDS and attends at once (one
 * launch); otherwise the two calls run in turn. The workspace (size from
 * gpkv_quest_decode_workspace_bytes) serves either. Errors: those of the two calls. */
size_t gpkv_quest_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int32_t max_blocks_per_seq,
                                         int32_t topk_blocks);
int gpkv_quest_decode(float* out, int32_t* topk_indices, const void* query,
                      const void* key_cache, const void* value_cache, const void* key_min,
                      const void* key_max, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                      int32_t topk_blocks, float scale, void* workspace, size_t workspace_bytes,
                      void* stream);

/* The Quest step with its cache write in one call (the KV-cache update sharing the
 * decode kernel's launch, [DSA] items 2-3): gpkv_reshape_and_cache_quest over the
 * batch's new tokens, then gpkv_quest_decode, for the decode-append case of
 * gpkv_paged_attention_decode_append (token b of key / value is sequence b's newest
 * token, at position context_lens[b] - 1; an in-pool slot_mapping[b] is that
 * position's slot; a slot outside the pool writes nothing). On the one-launch path
 * the workgroup of each (sequence, KV head) pair writes its head's part of the row
 * and folds it into the block's key min / max before it scores, selects and
 * attends; on the other path the write kernel runs first. The caches and the
 * metadata (modified in place at the written slots and their blocks) end bit for
 * bit as after the two calls, and topk_indices / out are those of gpkv_quest_decode
 * over them. The metadata must cover each sequence's earlier rows (the fold's
 * decode-append contract). key, value: [batch, num_kv_heads, head_dim] bf16;
 * slot_mapping: [batch] int64. Everything else as gpkv_quest_decode. */
int gpkv_quest_decode_append(float* out, int32_t* topk_indices, const void* query,
                             const void* key, const void* value, void* key_cache,
                             void* value_cache, void* key_min, void* key_max,
                             const int64_t* slot_mapping, const int32_t* block_tables,
                             const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int64_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t max_context_len, int32_t topk_blocks, float scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * FP8 KV cache. The pages name KV quantisation as the lever for long-context
 * decode, where the KV stream is the cost ([TL18] 2.5 item 3, 3.1 item 4); they
 * fix no format. Here: K and V caches hold OCP FP8 E4M3 codes (1 byte per
 * element: sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
 * largest finite 448; NaN = S.1111.111), with one float32 scale per KV head for
 * K (k_scale[H_kv]) and one for V (v_scale[H_kv]), in device memory, positive and
 * finite (precondition). The value of a code is code * scale.
 * Layouts are those of the bf16 calls with 1-byte elements:
 * key_cache, value_cache: [num_blocks, block_size, num_kv_heads, head_dim] uint8.
 * Workspaces: gpkv_paged_attention_workspace_bytes and
 * gpkv_sparse_attention_workspace_bytes give the sizes for these calls too.
 * --------------------------------------------------------------------------- */

/* ReshapeAndCache into E4M3 caches: the slot rule of gpkv_reshape_and_cache; each
 * element x of KV head g is stored as the E4M3 value nearest to
 * float32(x) * float32(1 / scale[g]) (a correctly rounded float32 division, then
 * one float32 product), ties to the even code, magnitudes past 448 saturating to
 * 448, NaN to 0x7F. key, value: [num_tokens, num_kv_heads, head_dim] bf16. */
int gpkv_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                               void* value_cache, const float* k_scale, const float* v_scale,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, void* stream);

/* gpkv_paged_attention_decode over E4M3 caches: K_t = code * k_scale[g],
 * V_t = code * v_scale[g]; query bf16, output float32 as in the bf16 call. */
int gpkv_paged_attention_decode_fp8(float* out, const void* query, const void* key_cache,
                                    const void* value_cache, const float* k_scale,
                                    const float* v_scale, const int32_t* block_tables,
                                    const int32_t* context_lens, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks,
                                    int32_t max_blocks_per_seq, int32_t max_context_len,
                                    float scale, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* The FP8 dense step in one call: gpkv_reshape_and_cache_fp8 over the batch's new
 * tokens followed by gpkv_paged_attention_decode_fp8, for the decode-append case of
 * gpkv_paged_attention_decode_append (token b of key / value is sequence b's newest
 * token, at position context_lens[b] - 1, and an in-pool slot_mapping[b] is that
 * position's slot). The combine kernel writes the token's codes (the FP8 write's
 * quantisation) and merges the token as one more unit with the values the cache then
 * holds, code * scale; the caches end bit for bit as after the two calls, attention
 * within the same tolerance. key, value: [batch, num_kv_heads, head_dim] bf16;
 * slot_mapping: [batch] int64; everything else as gpkv_paged_attention_decode_fp8. */
int gpkv_paged_attention_decode_fp8_append(float* out, const void* query, const void* key,
                                           const void* value, void* key_cache, void* value_cache,
                                           const float* k_scale, const float* v_scale,
                                           const int64_t* slot_mapping,
                                           const int32_t* block_tables,
                                           const int32_t* context_lens, int32_t batch,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int64_t num_blocks, int32_t max_blocks_per_seq,
                                           int32_t max_context_len, float scale, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* gpkv_sparse_paged_attention_decode over E4M3 caches (values as above). */
int gpkv_sparse_paged_attention_decode_fp8(float* out, const void* query, const void* key_cache,
                                           const void* value_cache, const float* k_scale,
                                           const float* v_scale, const int32_t* block_tables,
                                           const int32_t* context_lens,
                                           const int32_t* topk_indices, int32_t batch,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int64_t num_blocks, int32_t max_blocks_per_seq,
                                           int32_t max_context_len, int32_t topk_blocks,
                                           float scale, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* Quest over E4M3 caches ([ASC] "Quest Sparse Attention" with the FP8 cache above).
 * The pages give the metadata and the bound for one key format; for E4M3 keys this
 * library keeps, per (physical block, KV head, channel), the CODES of the smallest
 * and largest key code value over the block's valid rows (one byte each, half the
 * bf16 metadata's bytes). A key is code * k_scale[g] with k_scale[g] > 0, so these
 * are the keys' extremes divided by the scale. The block score is the Quest bound
 * over the code values:
 *   score(lb) = sum over h in group g, c of max(q[b,h,c] * val(key_min[pb,g,c]),
 *                                               q[b,h,c] * val(key_max[pb,g,c]))
 * in float64: the bound on the keys divided by k_scale[g], one positive factor for
 * every block of a KV head, so the selection (per KV head) is the same. A zero
 * extreme may be stored as either zero code (0x00 or 0x80); NaN codes are not
 * supported in the caches (they would order past +-448).
 * key_min, key_max: [num_blocks, num_kv_heads, head_dim] uint8 E4M3 codes.
 *
 * gpkv_quest_block_metadata_fp8: gpkv_quest_block_metadata over an E4M3 key_cache
 *   [num_blocks, block_size, num_kv_heads, head_dim] uint8, writing code metadata. */
int gpkv_quest_block_metadata_fp8(void* key_min, void* key_max, const void* key_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t batch, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int64_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  int32_t last_block_only, void* stream);

/* gpkv_reshape_and_cache_fp8 plus the fold of each written key row's codes into its
 * block's code metadata, as gpkv_reshape_and_cache_quest folds bf16 rows (row 0 of
 * a block starts its metadata afresh; a later row takes the min / max by value). */
int gpkv_reshape_and_cache_fp8_quest(const void* key, const void* value, void* key_cache,
                                     void* value_cache, const float* k_scale,
                                     const float* v_scale, void* key_min, void* key_max,
                                     const int64_t* slot_mapping, int32_t num_tokens,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int64_t num_blocks, void* stream);

/* gpkv_quest_select_topk over code metadata (the score above); the same workspace
 * (gpkv_quest_select_workspace_bytes), tie rule, output and errors. */
int gpkv_quest_select_topk_fp8(int32_t* topk_indices, const void* query, const void* key_min,
                               const void* key_max, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int32_t topk_blocks, void* workspace,
                               size_t workspace_bytes, void* stream);

/* gpkv_quest_decode over E4M3 caches and code metadata: the result of
 * gpkv_quest_select_topk_fp8 followed by gpkv_sparse_paged_attention_decode_fp8, in
 * one launch under the same rule as gpkv_quest_decode (with the pair's bytes at one
 * byte per element), else those two calls. Workspace from
 * gpkv_quest_decode_workspace_bytes. */
int gpkv_quest_decode_fp8(float* out, int32_t* topk_indices, const void* query,
                          const void* key_cache, const void* value_cache, const float* k_scale,
                          const float* v_scale, const void* key_min, const void* key_max,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int64_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_context_len,
                          int32_t topk_blocks, float scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/* gpkv_quest_decode_append over E4M3 caches: gpkv_reshape_and_cache_fp8_quest over the
 * batch's new tokens (key, value bf16 as there), then gpkv_quest_decode_fp8; on the
 * one-launch path each (sequence, KV head) workgroup quantises and writes its head's
 * part of the row and folds its codes before it scores. The caches end bit for bit
 * as after the two calls, the metadata equal by value. */
int gpkv_quest_decode_fp8_append(float* out, int32_t* topk_indices, const void* query,
                                 const void* key, const void* value, void* key_cache,
                                 void* value_cache, const float* k_scale, const float* v_scale,
                                 void* key_min, void* key_max, const int64_t* slot_mapping,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 int32_t topk_blocks, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Multi-token queries (varlen batches: [TL18] 2.7 continuous batching with
 * ragged lengths; 3.3 flattened queries with cu_seqlens and the causal mask
 * aligned to the right, item 4). Sequence b brings q_len_b =
 * cu_seqlens_q[b + 1] - cu_seqlens_q[b] query tokens: the newest q_len_b of its
 * context_lens[b] positions, whose K/V are already in the cache (written by
 * gpkv_reshape_and_cache). Query token j (0-based) of sequence b attends to the
 * positions t <= context_lens[b] - q_len_b + j:
 *   out[r, h, :] = sum_t p_t V_t, p = softmax_t(scale * q[r, h, :] . K_t),
 * r = cu_seqlens_q[b] + j, K_t / V_t of KV head h / G. A row that sees no
 * position (q_len_b > context_lens[b], j small) gets a zero row.
 * query: [total_q, num_q_heads, head_dim] bf16; out: same shape, float32.
 * cu_seqlens_q: [batch + 1] int32 in device memory, non-decreasing from 0 to
 *   total_q (a sequence whose offsets fall outside [0, total_q] or decrease is
 *   treated as empty). max_q_len: a host bound of every q_len_b (rows past it are
 *   not computed). Decode is the case q_len_b = 1.
 * workspace: at least gpkv_paged_attention_varlen_workspace_bytes(...) bytes;
 *   contents on entry ignored.
 * --------------------------------------------------------------------------- */
size_t gpkv_paged_attention_varlen_workspace_bytes(int32_t batch, int32_t total_q,
                                                   int32_t max_q_len, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t head_dim,
                                                   int32_t block_size, int32_t max_context_len);

int gpkv_paged_attention_varlen(float* out, const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* cu_seqlens_q,
                                int32_t batch, int32_t total_q, int32_t max_q_len,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* gpkv_paged_attention_varlen over E4M3 caches (KV quantisation, [TL18] 2.5 item 3
 * and 3.1 item 4, with the varlen rows of 2.7 / 3.3): key_cache / value_cache are
 * uint8 codes [num_blocks, block_size, num_kv_heads, head_dim] and k_scale /
 * v_scale float32 [num_kv_heads], read as code * scale (as for
 * gpkv_paged_attention_decode_fp8). Other arguments, the workspace size
 * (gpkv_paged_attention_varlen_workspace_bytes) and errors as for the bf16 call;
 * null scales give GPKV_ERR_NULL. */
int gpkv_paged_attention_varlen_fp8(float* out, const void* query, const void* key_cache,
                                    const void* value_cache, const float* k_scale,
                                    const float* v_scale, const int32_t* block_tables,
                                    const int32_t* context_lens, const int32_t* cu_seqlens_q,
                                    int32_t batch, int32_t total_q, int32_t max_q_len,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks,
                                    int32_t max_blocks_per_seq, int32_t max_context_len,
                                    float scale, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Static description of a status code. */
const char* gpkv_status_string(int status);

/* Detail of the last failing call on the calling thread ("" if none). */
const char* gpkv_last_error_message(void);

/* Tokens per split-KV work unit the attention calls pick for these sizes
 * (reported by benchmarks; the same value sizes the workspace). */
int32_t gpkv_split_tokens(int32_t batch, int32_t num_kv_heads, int32_t span_tokens);

#ifdef __cplusplus
}
#endif

#endif /* GPKV_H_ */
