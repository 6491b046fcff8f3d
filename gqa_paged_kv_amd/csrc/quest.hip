// Quest: per-block key min/max metadata, block scoring and Top-K selection.
//
// ["Ascend Kernel-to-Serving Pipeline", section "Quest Sparse Attention"]: score
// every logical block at low cost, keep the best topk_blocks blocks per KV head,
// skip blocks and tokens past the context, then run exact attention on the kept
// blocks only (that last step is the sparse path of paged_attention.hip).
//
// The low-cost score is the classic Quest bound: with per-channel key minimum
// and maximum of a block, max(q*kmin, q*kmax) bounds q*k for every key of the
// block, so the per-channel sum bounds q.k. The selection is per KV head; the
// group's query heads are summed. Because kmin <= kmax,
//   sum_h max(q_h*kmin, q_h*kmax) = kmax * sum_{q_h>0} q_h + kmin * sum_{q_h<0} q_h,
// so each (b, g) pre-reduces its queries once into two float64 vectors and a block
// costs 2*D float64 FMAs. Scores stay in float64 so near-equal blocks keep their
// exact order; ties go to the lower logical block. The _fp8 entry points do the same
// over E4M3 caches with metadata of codes (quest_select.h).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "gpkv_internal.h"
#include "quest_select.h"

namespace gpkv {

// ---------------------------------------------------------------------------
// Metadata: kmin / kmax over the valid rows of each referenced block
// ---------------------------------------------------------------------------

struct MetaParams {
  void* kmin;                // [NB, H_kv, D] bf16 (E4M3 codes: the FP8 kernel)
  void* kmax;
  const unsigned char* kc;   // [NB, bs, H_kv, D] bf16 (E4M3 codes)
  const int* bt;
  const int* ctx;
  long long NB;
  long long block_bytes;
  int row_bytes;             // H_kv * D * bytes per element
  int bs, max_blocks, max_ctx, last_only;
};

__device__ __forceinline__ unsigned pack_bf16_pair(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// One workgroup per (sequence, logical block). A token row of all KV heads is
// row_bytes contiguous bytes; threads take 16-byte chunks of it and split the
// block's rows among token groups, then merge the groups through LDS.
__global__ __launch_bounds__(256) void quest_meta_kernel(const MetaParams p) {
  __shared__ u32x4 red_min[256];
  __shared__ u32x4 red_max[256];
  const int b = blockIdx.y, tid = threadIdx.x;
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int nb = (ctx + p.bs - 1) / p.bs;
  const int lb = p.last_only ? nb - 1 : (int)blockIdx.x;
  if (lb < 0 || lb >= nb) return;
  const int pb = p.bt[(size_t)b * p.max_blocks + lb];
  if (pb < 0 || pb >= p.NB) return;
  const int n = min(p.bs, ctx - lb * p.bs);
  const unsigned char* blk = p.kc + (size_t)pb * (size_t)p.block_bytes;
  const int chunks = p.row_bytes / 16;
  const int cpp = chunks < 256 ? chunks : 256;
  const int groups = 256 / cpp;
  const int c_local = tid % cpp, tg = tid / cpp;

  for (int c0 = 0; c0 < chunks; c0 += cpp) {
    const int c = c0 + c_local;
    float mn[8], mx[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      mn[k] = INFINITY;
      mx[k] = -INFINITY;
    }
    if (tg < groups && c < chunks) {
      for (int t = tg; t < n; t += groups) {
        const u32x4 v = *(const u32x4*)(blk + (size_t)t * p.row_bytes + (size_t)c * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = bf16_lo(v[k]), hi = bf16_hi(v[k]);
          mn[2 * k] = fminf(mn[2 * k], lo);
          mx[2 * k] = fmaxf(mx[2 * k], lo);
          mn[2 * k + 1] = fminf(mn[2 * k + 1], hi);
          mx[2 * k + 1] = fmaxf(mx[2 * k + 1], hi);
        }
      }
    }
    __syncthreads();
    u32x4 pm, px;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      pm[k] = pack_bf16_pair(mn[2 * k], mn[2 * k + 1]);
      px[k] = pack_bf16_pair(mx[2 * k], mx[2 * k + 1]);
    }
    red_min[tid] = pm;
    red_max[tid] = px;
    __syncthreads();
    if (tg == 0 && c < chunks) {
      for (int gi = 1; gi < groups; ++gi) {
        const u32x4 om = red_min[gi * cpp + c_local], ox = red_max[gi * cpp + c_local];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          mn[2 * k] = fminf(mn[2 * k], bf16_lo(om[k]));
          mn[2 * k + 1] = fminf(mn[2 * k + 1], bf16_hi(om[k]));
          mx[2 * k] = fmaxf(mx[2 * k], bf16_lo(ox[k]));
          mx[2 * k + 1] = fmaxf(mx[2 * k + 1], bf16_hi(ox[k]));
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pm[k] = pack_bf16_pair(mn[2 * k], mn[2 * k + 1]);
        px[k] = pack_bf16_pair(mx[2 * k], mx[2 * k + 1]);
      }
      const size_t o = (size_t)pb * (p.row_bytes / 2) + (size_t)c * 8;
      *(u32x4*)((unsigned short*)p.kmin + o) = pm;
      *(u32x4*)((unsigned short*)p.kmax + o) = px;
    }
  }
}

// The same over an E4M3 key cache: a 16-byte chunk holds sixteen codes, compared
// as order bytes (e4m3_order_bytes: unsigned byte order is value order) and
// stored back as the codes of the extremes.
__global__ __launch_bounds__(256) void quest_meta_fp8_kernel(const MetaParams p) {
  __shared__ u32x4 red_min[256];
  __shared__ u32x4 red_max[256];
  const int b = blockIdx.y, tid = threadIdx.x;
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int nb = (ctx + p.bs - 1) / p.bs;
  const int lb = p.last_only ? nb - 1 : (int)blockIdx.x;
  if (lb < 0 || lb >= nb) return;
  const int pb = p.bt[(size_t)b * p.max_blocks + lb];
  if (pb < 0 || pb >= p.NB) return;
  const int n = min(p.bs, ctx - lb * p.bs);
  const unsigned char* blk = p.kc + (size_t)pb * (size_t)p.block_bytes;
  const int chunks = p.row_bytes / 16;
  const int cpp = chunks < 256 ? chunks : 256;
  const int groups = 256 / cpp;
  const int c_local = tid % cpp, tg = tid / cpp;

  for (int c0 = 0; c0 < chunks; c0 += cpp) {
    const int c = c0 + c_local;
    u32x4 mn = u32x4{~0u, ~0u, ~0u, ~0u}, mx = u32x4{0u, 0u, 0u, 0u};   // identities
    if (tg < groups && c < chunks) {
      for (int t = tg; t < n; t += groups) {
        const u32x4 v = *(const u32x4*)(blk + (size_t)t * p.row_bytes + (size_t)c * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const unsigned o = e4m3_order_bytes(v[k]);
          mn[k] = bytes_min(mn[k], o);
          mx[k] = bytes_max(mx[k], o);
        }
      }
    }
    __syncthreads();
    red_min[tid] = mn;
    red_max[tid] = mx;
    __syncthreads();
    if (tg == 0 && c < chunks) {   // group 0 holds row 0: every lane has a real extreme
      for (int gi = 1; gi < groups; ++gi) {
        const u32x4 om = red_min[gi * cpp + c_local], ox = red_max[gi * cpp + c_local];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          mn[k] = bytes_min(mn[k], om[k]);
          mx[k] = bytes_max(mx[k], ox[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mn[k] = e4m3_from_order_bytes(mn[k]);
        mx[k] = e4m3_from_order_bytes(mx[k]);
      }
      const size_t o = (size_t)pb * p.row_bytes + (size_t)c * 16;
      *(u32x4*)((unsigned char*)p.kmin + o) = mn;
      *(u32x4*)((unsigned char*)p.kmax + o) = mx;
    }
  }
}

// Two-kernel path, scoring: a workgroup covers kScoreBlocksPerWG consecutive logical
// blocks of one (b, g) and writes float64 scores (as their order-preserving keys).
template <int D, bool FP8>
__global__ __launch_bounds__(kSelectThreads) void quest_score_kernel(const ScoreParams p) {
  __shared__ double s_pos[D];
  __shared__ double s_neg[D];
  __shared__ unsigned short s_q[kMaxGroup * D];
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int nb = (ctx + p.bs - 1) / p.bs;
  const int lb0 = chunk * kScoreBlocksPerWG;
  if (lb0 >= nb || p.K >= nb) return;  // nothing to rank: every block is selected
  query_bounds<D>(p, b, g, s_q, s_pos, s_neg);
  unsigned long long* keys = (unsigned long long*)p.scores + ((size_t)b * p.Hkv + g) * p.max_blocks;
  score_blocks<D, FP8, kScoreUnroll>(p, g, nb, lb0,
                               [&](int lb) { return p.bt[(size_t)b * p.max_blocks + lb]; },
                               s_pos, s_neg,
                                [&](int lb, unsigned long long key) { keys[lb] = key; });
}

// Two-kernel path, scoring by whole metadata rows: a workgroup covers a chunk of
// logical blocks of one sequence for every KV head. The eight-lane groups of a
// block take its KV heads side by side, so a block's key-min row and key-max row
// (all KV heads, H_kv * D * 2 bytes each) are read whole and contiguously. Two
// passes of loads per workgroup (so twice the workgroups of four passes) measured
// fastest on MI355X: selection over 4 sequences x 2560 blocks 28.1 -> 25.4 us, over
// a ragged 256-sequence batch 25.3 -> 23.5 us; eight passes were slower (31.7 and
// 32.3 us).
constexpr int kRowScoreUnroll = 2;
constexpr int kMaxRowHeads = 32;

template <int D, bool FP8>
__global__ __launch_bounds__(kSelectThreads) void quest_score_rows_kernel(const ScoreParams p) {
  extern __shared__ double s_qb[];   // [H_kv][2][D + kQbPad]: positive / negative query sums
  constexpr int NV = D / 64;
  const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int Hkv = p.Hkv;
  const int bpp = (kSelectThreads / 8) / Hkv;        // blocks per pass
  const int lb0 = chunk * bpp * kRowScoreUnroll;
  const int sub = tid & 7, pair = tid >> 3;
  const int blk = pair / Hkv, g = pair % Hkv;
  const bool active = blk < bpp;
  // The chunk's table entries are requested together with the sequence's length
  // rather than after it (one dependent round trip fewer before the metadata
  // loads): the grid spans the longest context, whose entries the table holds, and
  // entries past this sequence's blocks are dropped once its length is known.
  const int max_nb = (p.max_ctx + p.bs - 1) / p.bs;
  int pbs[kRowScoreUnroll];
#pragma unroll
  for (int u = 0; u < kRowScoreUnroll; ++u) {
    const int lb = lb0 + u * bpp + blk;
    pbs[u] = (active && lb < max_nb) ? p.bt[(size_t)b * p.max_blocks + lb] : -1;
  }
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int nb = (ctx + p.bs - 1) / p.bs;
  if (lb0 >= nb || p.K >= nb) return;  // nothing to rank: every block is selected
  unsigned short* s_q = (unsigned short*)(s_qb + (size_t)Hkv * 2 * (D + kQbPad));   // [H_q][D] bf16
  stage_query<D>(p, b, 0, p.Hq, s_q);
  u32x4 mn[kRowScoreUnroll][NV], mx[kRowScoreUnroll][NV];
  bool ok[kRowScoreUnroll];
#pragma unroll
  for (int u = 0; u < kRowScoreUnroll; ++u) {
    const int lb = lb0 + u * bpp + blk;
    const int pb = lb < nb ? pbs[u] : -1;
    ok[u] = pb >= 0 && pb < p.NB;
    const size_t o = ((size_t)(ok[u] ? pb : 0) * Hkv + g) * D + (size_t)sub * 8;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      mn[u][v] = ok[u] ? meta_load8<FP8>(p.kmin, o + 64 * v) : u32x4{0, 0, 0, 0};
      mx[u][v] = ok[u] ? meta_load8<FP8>(p.kmax, o + 64 * v) : u32x4{0, 0, 0, 0};
    }
  }
  __syncthreads();
  for (int i = tid; i < Hkv * D; i += kSelectThreads) {
    const int gg = i / D, c = i % D;
    group_bounds<D>(s_q + (size_t)gg * p.G * D, p.G, c,
                    &s_qb[(gg * 2) * (D + kQbPad) + qb_index<D>(c)],
                    &s_qb[(gg * 2 + 1) * (D + kQbPad) + qb_index<D>(c)]);
  }
  __syncthreads();
  const double* s_pos = s_qb + (g * 2) * (D + kQbPad);
  const double* s_neg = s_qb + (g * 2 + 1) * (D + kQbPad);
  unsigned long long* keys = (unsigned long long*)p.scores + ((size_t)b * Hkv + g) * p.max_blocks;
#pragma unroll
  for (int u = 0; u < kRowScoreUnroll; ++u) {
    double acc = active ? bound_lane<D, FP8>(mn[u], mx[u], s_pos, s_neg, sub) : 0.0;
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    const int lb = lb0 + u * bpp + blk;
    if (active && lb < nb && sub == 0) keys[lb] = score_key(ok[u] ? acc : -INFINITY);
  }
}

// Two-kernel path, selection: one workgroup per (b, g) over the stored keys,
// staged in LDS when they fit.
struct TopkParams {
  int* out;                          // [B, H_kv, K]
  const unsigned long long* keys;    // [B, H_kv, max_blocks]
  const int* ctx;
  int Hkv, bs, max_blocks, max_ctx, K, lds_keys;
};

__global__ __launch_bounds__(kMaxSelectThreads) void quest_topk_kernel(const TopkParams p) {
  extern __shared__ unsigned long long s_key[];
  __shared__ SelectShared sh;
  const int g = blockIdx.x, b = blockIdx.y;
  const unsigned long long* keys = p.keys + ((size_t)b * p.Hkv + g) * p.max_blocks;
  // With keys in LDS, the keys of the longest context (lds_keys of them, at most
  // max_blocks) are requested together with the sequence's length rather than
  // after it; only the first n are ranked, the rest were not written by this step.
  for (int i = threadIdx.x; i < p.lds_keys; i += blockDim.x) s_key[i] = keys[i];
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int n = (ctx + p.bs - 1) / p.bs;
  int* out = p.out + ((size_t)b * p.Hkv + g) * p.K;
  if (select_all(n, p.K, out)) return;
  if (n <= p.lds_keys) {
    __syncthreads();
    radix_topk(n, p.K, [&](int i) { return s_key[i]; }, out, sh);
  } else {
    radix_topk(n, p.K, [&](int i) { return keys[i]; }, out, sh);
  }
}

// Fused path: one workgroup per (b, g) scores all its blocks into LDS keys and
// selects from them -- one launch, and the keys never leave the CU.
template <int D, bool FP8>
__global__ __launch_bounds__(kFusedThreads) void quest_select_fused_kernel(const ScoreParams p) {
  // Dynamic LDS: the keys of the sequence's blocks, then its block-table row.
  extern __shared__ unsigned long long s_key[];
  __shared__ double s_pos[D];
  __shared__ double s_neg[D];
  __shared__ unsigned short s_q[kMaxGroup * D];
  __shared__ SelectShared sh;
  const int g = blockIdx.x, b = blockIdx.y;
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int nb = (ctx + p.bs - 1) / p.bs;
  // One round of loads for the query group and the block-table row up to the
  // longest context (max_nb <= max_blocks: in bounds), issued without waiting for
  // this sequence's length, so the metadata loads below depend on LDS only.
  const int max_nb = (p.max_ctx + p.bs - 1) / p.bs;
  int* s_pb = (int*)(s_key + max_nb);
  stage_query<D>(p, b, g * p.G, p.G, s_q);
  for (int lb = threadIdx.x; lb < max_nb; lb += blockDim.x)
    s_pb[lb] = p.bt[(size_t)b * p.max_blocks + lb];
  int* out = p.out + ((size_t)b * p.Hkv + g) * p.K;
  if (select_all(nb, p.K, out)) return;
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += blockDim.x)
    group_bounds<D>(s_q, p.G, c, s_pos + qb_index<D>(c), s_neg + qb_index<D>(c));
  __syncthreads();
  for (int lb0 = 0; lb0 < nb; lb0 += (int)(blockDim.x >> 3) * kFusedUnroll)
    score_blocks<D, FP8, kFusedUnroll>(p, g, nb, lb0, [&](int lb) { return s_pb[lb]; }, s_pos,
                                       s_neg, [&](int lb, unsigned long long key) { s_key[lb] = key; });
  __syncthreads();
  radix_topk(nb, p.K, [&](int i) { return s_key[i]; }, out, sh);
}

static int check_quest(const char* fn, int B, int Hkv, int D, int bs, long long NB,
                       int max_blocks, int max_ctx) {
  if (B < 0 || Hkv <= 0 || NB < 0 || max_blocks <= 0 || max_ctx < 0)
    return fail(GPKV_ERR_SHAPE,
                "%s: batch=%d num_kv_heads=%d num_blocks=%lld max_blocks_per_seq=%d "
                "max_context_len=%d",
                fn, B, Hkv, NB, max_blocks, max_ctx);
  if (!supported_head_dim(D))
    return fail(GPKV_ERR_UNSUPPORTED, "%s: head_dim=%d (64 or 128)", fn, D);
  if (!supported_block_size(bs))
    return fail(GPKV_ERR_UNSUPPORTED, "%s: block_size=%d (16/32/64/128)", fn, bs);
  if ((long long)max_ctx > (long long)max_blocks * bs)
    return fail(GPKV_ERR_SHAPE, "%s: max_context_len=%d > max_blocks_per_seq*block_size=%lld",
                fn, max_ctx, (long long)max_blocks * bs);
  if (B > 65535 || Hkv > 65535)
    return fail(GPKV_ERR_SHAPE, "%s: batch or num_kv_heads above 65535", fn);
  return GPKV_OK;
}

static int meta_run(const char* fn, bool fp8, void* key_min, void* key_max,
                    const void* key_cache, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t batch, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks,
                    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t last_block_only,
                    void* stream) {
  int st = check_quest(fn, batch, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len);
  if (st) return st;
  if (batch == 0 || max_context_len == 0) return GPKV_OK;
  if (!key_min || !key_max || !key_cache || !block_tables || !context_lens)
    return fail(GPKV_ERR_NULL, "%s: null pointer argument", fn);
  MetaParams mp;
  mp.kmin = key_min;
  mp.kmax = key_max;
  mp.kc = (const unsigned char*)key_cache;
  mp.bt = block_tables;
  mp.ctx = context_lens;
  mp.NB = num_blocks;
  mp.row_bytes = num_kv_heads * head_dim * (fp8 ? 1 : 2);
  mp.block_bytes = (long long)block_size * mp.row_bytes;
  mp.bs = block_size;
  mp.max_blocks = max_blocks_per_seq;
  mp.max_ctx = max_context_len;
  mp.last_only = last_block_only ? 1 : 0;
  const int max_nb = (max_context_len + block_size - 1) / block_size;
  const dim3 grid(last_block_only ? 1 : max_nb, batch);
  if (fp8)
    quest_meta_fp8_kernel<<<grid, dim3(256), 0, (hipStream_t)stream>>>(mp);
  else
    quest_meta_kernel<<<grid, dim3(256), 0, (hipStream_t)stream>>>(mp);
  return check_launch(fn);
}

template <bool FP8>
static int select_run(const char* fn, int32_t* topk_indices, const void* query,
                      const void* key_min, const void* key_max, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                      int32_t topk_blocks, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int st = check_quest(fn, batch, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len);
  if (st) return st;
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(GPKV_ERR_SHAPE, "%s: num_q_heads=%d is not a positive multiple of num_kv_heads=%d",
                fn, num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > kMaxGroup)
    return fail(GPKV_ERR_UNSUPPORTED, "%s: group size %d > %d", fn, num_q_heads / num_kv_heads,
                kMaxGroup);
  if (topk_blocks < 1) return fail(GPKV_ERR_SHAPE, "%s: topk_blocks=%d < 1", fn, topk_blocks);
  if (batch == 0) return GPKV_OK;
  if (!topk_indices || !query || !key_min || !key_max || !block_tables || !context_lens)
    return fail(GPKV_ERR_NULL, "%s: null pointer argument", fn);
  const size_t need = gpkv_quest_select_workspace_bytes(batch, num_kv_heads, max_blocks_per_seq);
  if (!workspace || workspace_bytes < need)
    return fail(GPKV_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  hipStream_t s = (hipStream_t)stream;
  const int max_nb = (max_context_len + block_size - 1) / block_size;
  ScoreParams sp;
  sp.scores = (double*)workspace;
  sp.out = topk_indices;
  sp.q = (const unsigned short*)query;
  sp.kmin = key_min;
  sp.kmax = key_max;
  sp.bt = block_tables;
  sp.ctx = context_lens;
  sp.NB = num_blocks;
  sp.Hq = num_q_heads;
  sp.Hkv = num_kv_heads;
  sp.G = num_q_heads / num_kv_heads;
  sp.bs = block_size;
  sp.max_blocks = max_blocks_per_seq;
  sp.max_ctx = max_context_len;
  sp.K = topk_blocks;
  // Enough (b, g) pairs to spread over the GPU and keys that fit in LDS: one fused
  // launch. Otherwise score with a grid over blocks first, then select.
  // GPKV_QUEST_SELECT_PATH=fused|two_kernel overrides the choice (tuning aid).
  const char* forced = getenv("GPKV_QUEST_SELECT_PATH");
  // Measured on MI355X: one fused launch wins for many (b, g) pairs with long
  // tables (it skips the round trip of the keys); short tables and few pairs are
  // faster with the grid-wide scoring kernel.
  bool fused = (long long)batch * num_kv_heads >= 128 && max_nb >= 512;
  if (forced && strcmp(forced, "fused") == 0) fused = true;
  if (forced && strcmp(forced, "two_kernel") == 0) fused = false;
  if (fused && max_nb <= kMaxFusedBlocks) {
    const size_t lds = (size_t)(max_nb > 0 ? max_nb : 1) * (sizeof(unsigned long long) + sizeof(int));
    // Threads so that one round of kFusedUnroll passes covers the longest table.
    int threads = kSelectThreads;
    while (threads < kFusedThreads && threads / 8 * kFusedUnroll < max_nb) threads <<= 1;
    const dim3 grid(num_kv_heads, batch);
    if (head_dim == 128)
      quest_select_fused_kernel<128, FP8><<<grid, dim3(threads), lds, s>>>(sp);
    else
      quest_select_fused_kernel<64, FP8><<<grid, dim3(threads), lds, s>>>(sp);
    return check_launch(fn);
  }
  const size_t row_lds = (size_t)num_kv_heads * 2 * (head_dim + kQbPad) * sizeof(double) +
                         (size_t)num_q_heads * head_dim * sizeof(unsigned short);
  if (max_nb > 0 && num_kv_heads <= kMaxRowHeads && row_lds <= 48 * 1024) {
    const int per_wg = (kSelectThreads / 8) / num_kv_heads * kRowScoreUnroll;
    const dim3 grid((max_nb + per_wg - 1) / per_wg, batch);
    if (head_dim == 128)
      quest_score_rows_kernel<128, FP8><<<grid, dim3(kSelectThreads), row_lds, s>>>(sp);
    else
      quest_score_rows_kernel<64, FP8><<<grid, dim3(kSelectThreads), row_lds, s>>>(sp);
    st = check_launch(fn);
    if (st) return st;
  } else if (max_nb > 0) {
    const dim3 grid((max_nb + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG, num_kv_heads, batch);
    if (head_dim == 128)
      quest_score_kernel<128, FP8><<<grid, dim3(kSelectThreads), 0, s>>>(sp);
    else
      quest_score_kernel<64, FP8><<<grid, dim3(kSelectThreads), 0, s>>>(sp);
    st = check_launch(fn);
    if (st) return st;
  }
  TopkParams tp;
  tp.out = topk_indices;
  tp.keys = (const unsigned long long*)workspace;
  tp.ctx = context_lens;
  tp.Hkv = num_kv_heads;
  tp.bs = block_size;
  tp.max_blocks = max_blocks_per_seq;
  tp.max_ctx = max_context_len;
  tp.K = topk_blocks;
  tp.lds_keys = max_nb <= kMaxLdsKeys ? max_nb : 0;
  const size_t lds = (size_t)(tp.lds_keys > 0 ? tp.lds_keys : 1) * sizeof(unsigned long long);
  // Few (sequence, KV head) pairs leave most CUs idle: give each pair's select up
  // to 1024 threads (about two keys each) so its radix passes are shorter.
  int topk_threads = kSelectThreads;
  const long long topk_pairs = (long long)batch * num_kv_heads;
  while (topk_threads < kMaxSelectThreads && topk_pairs * 4 <= balanced_capacity() &&
         2 * topk_threads <= max_nb)
    topk_threads <<= 1;
  quest_topk_kernel<<<dim3(num_kv_heads, batch), dim3(topk_threads), lds, s>>>(tp);
  return check_launch(fn);
}

}  // namespace gpkv

using namespace gpkv;

extern "C" int gpkv_quest_block_metadata(void* key_min, void* key_max, const void* key_cache,
                                         const int32_t* block_tables,
                                         const int32_t* context_lens, int32_t batch,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int64_t num_blocks,
                                         int32_t max_blocks_per_seq, int32_t max_context_len,
                                         int32_t last_block_only, void* stream) {
  clear_error();
  return meta_run("quest_block_metadata", false, key_min, key_max, key_cache, block_tables,
                  context_lens, batch, num_kv_heads, head_dim, block_size, num_blocks,
                  max_blocks_per_seq, max_context_len, last_block_only, stream);
}

extern "C" int gpkv_quest_block_metadata_fp8(void* key_min, void* key_max, const void* key_cache,
                                             const int32_t* block_tables,
                                             const int32_t* context_lens, int32_t batch,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int64_t num_blocks,
                                             int32_t max_blocks_per_seq, int32_t max_context_len,
                                             int32_t last_block_only, void* stream) {
  clear_error();
  return meta_run("quest_block_metadata_fp8", true, key_min, key_max, key_cache, block_tables,
                  context_lens, batch, num_kv_heads, head_dim, block_size, num_blocks,
                  max_blocks_per_seq, max_context_len, last_block_only, stream);
}

extern "C" size_t gpkv_quest_select_workspace_bytes(int32_t batch, int32_t num_kv_heads,
                                                    int32_t max_blocks_per_seq) {
  if (batch < 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0) return 0;
  return (size_t)batch * num_kv_heads * max_blocks_per_seq * sizeof(double);
}

extern "C" int gpkv_quest_select_topk(int32_t* topk_indices, const void* query,
                                      const void* key_min, const void* key_max,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      int32_t topk_blocks, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  clear_error();
  return select_run<false>("quest_select_topk", topk_indices, query, key_min, key_max,
                           block_tables, context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                           block_size, num_blocks, max_blocks_per_seq, max_context_len,
                           topk_blocks, workspace, workspace_bytes, stream);
}

extern "C" int gpkv_quest_select_topk_fp8(int32_t* topk_indices, const void* query,
                                          const void* key_min, const void* key_max,
                                          const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t batch,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          int64_t num_blocks, int32_t max_blocks_per_seq,
                                          int32_t max_context_len, int32_t topk_blocks,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return select_run<true>("quest_select_topk_fp8", topk_indices, query, key_min, key_max,
                          block_tables, context_lens, batch, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, max_blocks_per_seq, max_context_len, topk_blocks,
                          workspace, workspace_bytes, stream);
}
