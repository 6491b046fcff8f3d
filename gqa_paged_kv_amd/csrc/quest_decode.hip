// The Quest decode step in one call: block selection and sparse attention over the
// selection, in one launch when the (sequence, KV head) pairs fill the GPU.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "attention.h"
#include "quest_select.h"

namespace gpkv {

// ["Ascend Kernel-to-Serving Pipeline", section "test results and interpretation",
// item 4]: beyond the KV bytes it skips, the sparse path pays for scoring, Top-K,
// indexing and the scheduling of several kernels. When the batch's
// (sequence, KV head) pairs take at most one workgroup per CU, one workgroup per
// pair does all of it: it stages the pair's block-table row once, scores every
// block into LDS keys, radix-selects the Top-K ids into LDS (and writes them
// out), then its eight waves attend over the selected blocks through the staged
// table, and their partial rows meet in LDS as on the direct sparse path. The
// selection and the attention are those of quest_select_topk and
// sparse_paged_attention_decode.
constexpr int kQuestWaves = kFusedThreads / 64;

struct QuestDecodeParams {
  ScoreParams sp;            // sp.out: topk_indices [B, H_kv, K]
  AttnCommon c;
  float* out;                // [B, H_q, D] fp32
  int max_nb;                // table entries the dynamic LDS holds
  // Decode append (slots non-null): the workgroup of (b, g) first writes KV head g's
  // part of sequence b's new token into the cache and folds it into the block's key
  // min / max, so that its scores and its attention see the written cache. Only
  // that workgroup touches head g's part of the row and of the metadata.
  const long long* slots;    // [B]
  long long num_slots;       // NB * bs
  const unsigned short* knew;   // [B, H_kv, D] bf16
  const unsigned short* vnew;
  void* kc_w;                // the caches and metadata (bf16, or E4M3 codes)
  void* vc_w;
  void* kmin_w;
  void* kmax_w;
};

// FP8: E4M3 caches with per-KV-head scales (c.k_scale, c.v_scale) and E4M3
// metadata; the new token is quantised as the FP8 write path does it.
template <int D, bool FP8>
__global__ __launch_bounds__(kFusedThreads) void quest_decode_fused_kernel(const QuestDecodeParams p) {
  // Dynamic LDS: keys [max_nb, padded to 2], block-table row [max_nb, padded to 4],
  // then the waves' partial rows [kQuestWaves][G][D] (16-byte aligned).
  extern __shared__ __align__(16) unsigned long long s_dyn[];
  __shared__ double s_pos[D];
  __shared__ double s_neg[D];
  __shared__ unsigned short s_q[kMaxGroup * D];
  __shared__ SelectShared sh;
  __shared__ int s_sel[kDirTab];
  __shared__ float s_lse[kQuestWaves * kMaxGroup];
  const ScoreParams& sp = p.sp;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int G = sp.G, bs = sp.bs, K = sp.K;
  const int ctx = clamp_ctx(sp.ctx[b], sp.max_ctx);
  const int nb = (ctx + bs - 1) / bs;
  unsigned long long* s_key = s_dyn;
  int* s_pb = (int*)(s_key + ((p.max_nb + 1) & ~1));
  float* s_o = (float*)(s_pb + ((p.max_nb + 3) & ~3));
  int* out_ids = sp.out + ((size_t)b * sp.Hkv + g) * K;

  // Selection (as quest_select_fused_kernel, into LDS). The table row is staged
  // up to the longest context and the query group unconditionally, so neither
  // waits for this sequence's length (max_nb <= max_blocks: in bounds).
  for (int lb = tid; lb < p.max_nb; lb += kFusedThreads)
    s_pb[lb] = sp.bt[(size_t)b * sp.max_blocks + lb];
  const bool all = K >= nb;
  stage_query<D>(sp, b, g * G, G, s_q);
  if (p.slots != nullptr) {
    const long long s = p.slots[b];
    if (s >= 0 && s < p.num_slots) {
      if constexpr (FP8)
        store_new_token_fp8<D>(p.knew, p.vnew, (unsigned char*)p.kc_w, (unsigned char*)p.vc_w,
                               (unsigned char*)p.kmin_w, (unsigned char*)p.kmax_w, p.c.k_scale,
                               p.c.v_scale, s, bs, sp.Hkv, b, g, tid, kFusedThreads);
      else
        store_new_token<D>(p.knew, p.vnew, (unsigned short*)p.kc_w, (unsigned short*)p.vc_w,
                           (unsigned short*)p.kmin_w, (unsigned short*)p.kmax_w, s, bs, sp.Hkv, b,
                           g, tid, kFusedThreads);
    }
  }
  __syncthreads();   // (the barrier also orders the new token's stores before every read)
  if (all) {
    for (int i = tid; i < K; i += kFusedThreads) {
      out_ids[i] = i < nb ? i : -1;
      if (i < nb) s_sel[i] = i;
    }
  } else {
    for (int c = tid; c < D; c += kFusedThreads)
      group_bounds<D>(s_q, G, c, s_pos + qb_index<D>(c), s_neg + qb_index<D>(c));
    __syncthreads();
    for (int lb0 = 0; lb0 < nb; lb0 += (kFusedThreads >> 3) * kFusedUnroll)
      score_blocks<D, FP8, kFusedUnroll>(sp, g, nb, lb0, [&](int lb) { return s_pb[lb]; }, s_pos,
                                         s_neg, [&](int lb, unsigned long long key) { s_key[lb] = key; });
    __syncthreads();
    radix_topk(nb, K, [&](int i) { return s_key[i]; }, s_sel, sh);
    __syncthreads();
    for (int i = tid; i < K; i += kFusedThreads) out_ids[i] = s_sel[i];
  }
  __syncthreads();

  // Attention over the min(K, nb) selected blocks (ascending ids, all valid): wave
  // w takes a contiguous share of the 32-token tiles.
  const int spb = bs >> 4;
  const int n_sub = (K < nb ? K : nb) * spb;
  const int n_tiles = (n_sub + 1) >> 1;
  const int ta = wave * n_tiles / kQuestWaves, tb = (wave + 1) * n_tiles / kQuestWaves;
  const int ub = 2 * ta;
  const int ue = 2 * tb < n_sub ? 2 * tb : n_sub;
  auto desc = [&](int u, int& pb, int& row0, int& nv) {
    const int v = ub + u;
    const int blk = v / spb;
    row0 = (v - blk * spb) * 16;
    const int id = s_sel[blk];
    const int x = s_pb[id];
    const bool ok = x >= 0 && x < sp.NB;
    int n = ctx - (id * bs + row0);
    n = n < 0 ? 0 : (n > 16 ? 16 : n);
    if (!ok) n = 0;
    nv = uniform(n);
    pb = uniform(ok ? x : 0);
  };
  const int rr = tid & 15;
  RowTiles<1> rows;
  rows.q[0] = rr < G ? p.c.q + ((size_t)b * p.c.Hq + (size_t)g * G + rr) * D : nullptr;
  rows.n_rows[0] = G;
  rows.limit[0] = 0;
  rows.o[0] = s_o + wave * G * D;
  rows.lse[0] = s_lse + wave * kMaxGroup;
  attend_head<D, FP8, false, 1>(p.c, g, ue > ub ? ue - ub : 0, desc, 0, rows);
  __syncthreads();

  // out = sum_w 2^(lse_w - M) O_w / sum_w 2^(lse_w - M); no valid token: zeros.
  float* dst = p.out + ((size_t)b * p.c.Hq + (size_t)g * G) * D;
  for (int i = tid; i < G * (D / 4); i += kFusedThreads) {
    const int h = i / (D / 4), d = 4 * (i - h * (D / 4));
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kQuestWaves; ++w) m = fmaxf(m, s_lse[w * kMaxGroup + h]);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kQuestWaves; ++w) {
        const float wt = __builtin_amdgcn_exp2f(s_lse[w * kMaxGroup + h] - m);
        acc += wt * *(const f32x4*)(s_o + (w * G + h) * D + d);
        den += wt;
      }
      acc *= 1.f / den;
    }
    *(f32x4*)(dst + (size_t)h * D + d) = acc;
  }
}

}  // namespace gpkv

using namespace gpkv;

// One launch for the Quest decode step when the (sequence, KV head) pairs fill
// between half of the CUs and all of them (one 512-thread workgroup per CU: the
// attention's registers leave room for no second one), or when each pair reads
// little; otherwise the selection and the sparse attention calls in turn, sharing
// the workspace.
// GPKV_QUEST_DECODE_PATH=fused|separate forces the choice (tuning and test switch).
extern "C" size_t gpkv_quest_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t block_size,
                                                    int32_t max_blocks_per_seq,
                                                    int32_t topk_blocks) {
  const size_t a = gpkv_sparse_attention_workspace_bytes(batch, num_q_heads, num_kv_heads,
                                                         head_dim, block_size, topk_blocks);
  if (a == 0 || max_blocks_per_seq <= 0) return 0;
  const size_t b = gpkv_quest_select_workspace_bytes(batch, num_kv_heads, max_blocks_per_seq);
  return a > b ? a : b;
}

// Decode append inputs of gpkv_quest_decode_append and its FP8 variant.
struct QuestAppend {
  const void* key;
  const void* value;
  const int64_t* slots;
};

// FP8 caches and metadata (E4M3) with their per-KV-head scales.
struct QuestFp8 {
  const float* k_scale;
  const float* v_scale;
};

static int quest_decode_run(const char* fn, float* out, int32_t* topk_indices, const void* query,
                            const void* key_cache, const void* value_cache, const void* key_min,
                            const void* key_max, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, int32_t topk_blocks, float scale,
                            void* workspace, size_t workspace_bytes, void* stream,
                            const QuestAppend* app, const QuestFp8* fp8) {
  int st = check_common(fn, batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_blocks_per_seq, max_context_len);
  if (st) return st;
  if (topk_blocks < 1) return fail(GPKV_ERR_SHAPE, "%s: topk_blocks=%d < 1", fn, topk_blocks);
  if ((long long)topk_blocks * block_size > (1LL << 30))
    return fail(GPKV_ERR_SHAPE, "%s: token span too large", fn);
  if (batch == 0) return GPKV_OK;
  if (!out || !topk_indices || !query || !key_cache || !value_cache || !key_min || !key_max ||
      !block_tables || !context_lens || (app && (!app->key || !app->value || !app->slots)) ||
      (fp8 && (!fp8->k_scale || !fp8->v_scale)))
    return fail(GPKV_ERR_NULL, "%s: null pointer argument", fn);
  const size_t need = gpkv_quest_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                        block_size, max_blocks_per_seq,
                                                        topk_blocks);
  if (!workspace || workspace_bytes < need)
    return fail(GPKV_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn,
                workspace ? workspace_bytes : (size_t)0, need);

  const int G = num_q_heads / num_kv_heads;
  const int max_nb = (max_context_len + block_size - 1) / block_size;
  const size_t lds = (size_t)((max_nb + 1) & ~1) * sizeof(unsigned long long) +
                     (size_t)((max_nb + 3) & ~3) * sizeof(int) +
                     (size_t)kQuestWaves * G * head_dim * sizeof(float);
  const long long pairs = (long long)batch * num_kv_heads;
  const long long cus = balanced_capacity();
  const bool fits = topk_blocks <= kDirTab && max_nb <= kMaxFusedBlocks && lds <= 64 * 1024;
  // One workgroup per pair does the pair's whole step serially, so it pays when
  // the pairs fill the CUs, or when a pair's whole read (its metadata rows, then
  // its selected K/V) is small enough that the serial chain is shorter than the
  // two calls' four launches. Measured on MI355X: two 5-block pairs 11.7 us in one
  // launch against 21.2 us as two calls; sixteen 2560-block pairs 111 us against
  // 38 us.
  const int eb = fp8 ? 1 : 2;   // bytes per cached element and per metadata channel
  const long long pair_bytes =
      (long long)max_nb * 2 * head_dim * eb +
      (long long)(topk_blocks < max_nb ? topk_blocks : max_nb) * block_size * 2 * head_dim * eb;
  bool fused = fits && pairs <= cus && (2 * pairs > cus || pair_bytes <= 256 * 1024);
  const char* forced = getenv("GPKV_QUEST_DECODE_PATH");
  if (forced && strcmp(forced, "fused") == 0) fused = fits;
  if (forced && strcmp(forced, "separate") == 0) fused = false;
  if (!fused && fp8) {
    if (app) {   // the write (and metadata fold) first, then the two calls
      st = gpkv_reshape_and_cache_fp8_quest(app->key, app->value, (void*)key_cache,
                                            (void*)value_cache, fp8->k_scale, fp8->v_scale,
                                            (void*)key_min, (void*)key_max, app->slots, batch,
                                            num_kv_heads, head_dim, block_size, num_blocks, stream);
      if (st) return st;
    }
    st = gpkv_quest_select_topk_fp8(topk_indices, query, key_min, key_max, block_tables,
                                    context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                    block_size, num_blocks, max_blocks_per_seq, max_context_len,
                                    topk_blocks, workspace, workspace_bytes, stream);
    if (st) return st;
    return gpkv_sparse_paged_attention_decode_fp8(
        out, query, key_cache, value_cache, fp8->k_scale, fp8->v_scale, block_tables,
        context_lens, topk_indices, batch, num_q_heads, num_kv_heads, head_dim, block_size,
        num_blocks, max_blocks_per_seq, max_context_len, topk_blocks, scale, workspace,
        workspace_bytes, stream);
  }
  if (!fused) {
    if (app) {   // the write (and metadata fold) first, then the two calls
      st = gpkv_reshape_and_cache_quest(app->key, app->value, (void*)key_cache, (void*)value_cache,
                                        (void*)key_min, (void*)key_max, app->slots, batch,
                                        num_kv_heads, head_dim, block_size, num_blocks, stream);
      if (st) return st;
    }
    st = gpkv_quest_select_topk(topk_indices, query, key_min, key_max, block_tables,
                                context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                block_size, num_blocks, max_blocks_per_seq, max_context_len,
                                topk_blocks, workspace, workspace_bytes, stream);
    if (st) return st;
    return gpkv_sparse_paged_attention_decode(out, query, key_cache, value_cache, block_tables,
                                              context_lens, topk_indices, batch, num_q_heads,
                                              num_kv_heads, head_dim, block_size, num_blocks,
                                              max_blocks_per_seq, max_context_len, topk_blocks,
                                              scale, workspace, workspace_bytes, stream);
  }
  QuestDecodeParams qp;
  ScoreParams& sp = qp.sp;
  sp.scores = nullptr;
  sp.out = topk_indices;
  sp.q = (const unsigned short*)query;
  sp.kmin = key_min;
  sp.kmax = key_max;
  sp.bt = block_tables;
  sp.ctx = context_lens;
  sp.NB = num_blocks;
  sp.Hq = num_q_heads;
  sp.Hkv = num_kv_heads;
  sp.G = G;
  sp.bs = block_size;
  sp.max_blocks = max_blocks_per_seq;
  sp.max_ctx = max_context_len;
  sp.K = topk_blocks;
  AttnCommon& c = qp.c;
  c.q = (const unsigned short*)query;
  c.kc = (const unsigned char*)key_cache;
  c.vc = (const unsigned char*)value_cache;
  c.k_scale = fp8 ? fp8->k_scale : nullptr;
  c.v_scale = fp8 ? fp8->v_scale : nullptr;
  c.row_bytes = num_kv_heads * head_dim * eb;
  c.block_bytes = (long long)block_size * c.row_bytes;
  c.Hq = num_q_heads;
  c.Hkv = num_kv_heads;
  c.G = G;
  c.bs = block_size;
  c.qk_scale_log2 = scale * 1.4426950408889634f;
  qp.out = out;
  qp.max_nb = max_nb;
  qp.slots = app ? (const long long*)app->slots : nullptr;
  qp.num_slots = (long long)num_blocks * block_size;
  qp.knew = app ? (const unsigned short*)app->key : nullptr;
  qp.vnew = app ? (const unsigned short*)app->value : nullptr;
  qp.kc_w = (void*)key_cache;   // written only by the append calls
  qp.vc_w = (void*)value_cache;
  qp.kmin_w = (void*)key_min;
  qp.kmax_w = (void*)key_max;
  const dim3 grid(num_kv_heads, batch), block(kFusedThreads);
  hipStream_t s = (hipStream_t)stream;
  if (head_dim == 128 && fp8)
    quest_decode_fused_kernel<128, true><<<grid, block, lds, s>>>(qp);
  else if (head_dim == 128)
    quest_decode_fused_kernel<128, false><<<grid, block, lds, s>>>(qp);
  else if (fp8)
    quest_decode_fused_kernel<64, true><<<grid, block, lds, s>>>(qp);
  else
    quest_decode_fused_kernel<64, false><<<grid, block, lds, s>>>(qp);
  return check_launch(fn);
}

extern "C" int gpkv_quest_decode(float* out, int32_t* topk_indices, const void* query,
                                 const void* key_cache, const void* value_cache,
                                 const void* key_min, const void* key_max,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 int32_t topk_blocks, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  clear_error();
  return quest_decode_run("quest_decode", out, topk_indices, query, key_cache, value_cache,
                          key_min, key_max, block_tables, context_lens, batch, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                          max_context_len, topk_blocks, scale, workspace, workspace_bytes, stream,
                          nullptr, nullptr);
}

extern "C" int gpkv_quest_decode_append(float* out, int32_t* topk_indices, const void* query,
                                        const void* key, const void* value, void* key_cache,
                                        void* value_cache, void* key_min, void* key_max,
                                        const int64_t* slot_mapping, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t batch,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                        int32_t max_blocks_per_seq, int32_t max_context_len,
                                        int32_t topk_blocks, float scale, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  clear_error();
  QuestAppend app{key, value, slot_mapping};
  return quest_decode_run("quest_decode_append", out, topk_indices, query, key_cache,
                          value_cache, key_min, key_max, block_tables, context_lens, batch,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                          max_blocks_per_seq, max_context_len, topk_blocks, scale, workspace,
                          workspace_bytes, stream, &app, nullptr);
}

extern "C" int gpkv_quest_decode_fp8(float* out, int32_t* topk_indices, const void* query,
                                     const void* key_cache, const void* value_cache,
                                     const float* k_scale, const float* v_scale,
                                     const void* key_min, const void* key_max,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     int32_t topk_blocks, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  clear_error();
  QuestFp8 f{k_scale, v_scale};
  return quest_decode_run("quest_decode_fp8", out, topk_indices, query, key_cache, value_cache,
                          key_min, key_max, block_tables, context_lens, batch, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                          max_context_len, topk_blocks, scale, workspace, workspace_bytes, stream,
                          nullptr, &f);
}

extern "C" int gpkv_quest_decode_fp8_append(float* out, int32_t* topk_indices, const void* query,
                                            const void* key, const void* value, void* key_cache,
                                            void* value_cache, const float* k_scale,
                                            const float* v_scale, void* key_min, void* key_max,
                                            const int64_t* slot_mapping,
                                            const int32_t* block_tables,
                                            const int32_t* context_lens, int32_t batch,
                                            int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t block_size,
                                            int64_t num_blocks, int32_t max_blocks_per_seq,
                                            int32_t max_context_len, int32_t topk_blocks,
                                            float scale, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  clear_error();
  QuestAppend app{key, value, slot_mapping};
  QuestFp8 f{k_scale, v_scale};
  return quest_decode_run("quest_decode_fp8_append", out, topk_indices, query, key_cache,
                          value_cache, key_min, key_max, block_tables, context_lens, batch,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                          max_blocks_per_seq, max_context_len, topk_blocks, scale, workspace,
                          workspace_bytes, stream, &app, &f);
}
