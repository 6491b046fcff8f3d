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
// exact order; ties go to the lower logical block.
#include <math.h>

#include "gpkv_internal.h"

namespace gpkv {

// ---------------------------------------------------------------------------
// Metadata: kmin / kmax over the valid rows of each referenced block
// ---------------------------------------------------------------------------

struct MetaParams {
  unsigned short* kmin;      // [NB, H_kv, D] bf16
  unsigned short* kmax;
  const unsigned char* kc;   // [NB, bs, H_kv, D] bf16
  const int* bt;
  const int* ctx;
  long long NB;
  long long block_bytes;
  int row_bytes;             // H_kv * D * 2
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
      *(u32x4*)(p.kmin + o) = pm;
      *(u32x4*)(p.kmax + o) = px;
    }
  }
}

// ---------------------------------------------------------------------------
// Scores: one float64 per (sequence, KV head, logical block)
// ---------------------------------------------------------------------------

constexpr int kScoreBlocksPerWG = 64;

struct ScoreParams {
  double* scores;              // [B, H_kv, max_blocks]
  const unsigned short* q;     // [B, H_q, D]
  const unsigned short* kmin;  // [NB, H_kv, D]
  const unsigned short* kmax;
  const int* bt;
  const int* ctx;
  long long NB;
  int Hq, Hkv, G, bs, max_blocks, max_ctx;
};

// Eight lanes score one block (D/8 channels each) and merge with xor shuffles;
// a workgroup covers 64 consecutive logical blocks of one (b, g).
template <int D>
__global__ __launch_bounds__(256) void quest_score_kernel(const ScoreParams p) {
  constexpr int CH = D / 8;
  __shared__ double s_pos[D];
  __shared__ double s_neg[D];
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int nb = (ctx + p.bs - 1) / p.bs;
  const int lb0 = chunk * kScoreBlocksPerWG;
  if (lb0 >= nb) return;

  for (int c = tid; c < D; c += 256) {
    double pos = 0.0, neg = 0.0;
    const unsigned short* qh = p.q + ((size_t)b * p.Hq + (size_t)g * p.G) * D + c;
    for (int h = 0; h < p.G; ++h) {
      const double v = (double)__uint_as_float((unsigned)qh[(size_t)h * D] << 16);
      if (v > 0.0)
        pos += v;
      else
        neg += v;
    }
    s_pos[c] = pos;
    s_neg[c] = neg;
  }
  __syncthreads();

  const int sub = tid & 7, slot = tid >> 3;
  for (int it = 0; it < kScoreBlocksPerWG / 32; ++it) {
    const int lb = lb0 + it * 32 + slot;
    int pb = -1;
    if (lb < nb) pb = p.bt[(size_t)b * p.max_blocks + lb];
    const bool ok = lb < nb && pb >= 0 && pb < p.NB;
    double acc = 0.0;
    if (ok) {
      const size_t o = ((size_t)pb * p.Hkv + g) * D + (size_t)sub * CH;
      const u32x4* mn = (const u32x4*)(p.kmin + o);
      const u32x4* mx = (const u32x4*)(p.kmax + o);
#pragma unroll
      for (int v = 0; v < CH / 8; ++v) {
        const u32x4 a = mn[v], c4 = mx[v];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int ch = sub * CH + v * 8 + 2 * k;
          acc = fma((double)bf16_lo(c4[k]), s_pos[ch], acc);
          acc = fma((double)bf16_lo(a[k]), s_neg[ch], acc);
          acc = fma((double)bf16_hi(c4[k]), s_pos[ch + 1], acc);
          acc = fma((double)bf16_hi(a[k]), s_neg[ch + 1], acc);
        }
      }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (lb < nb && sub == 0)
      p.scores[((size_t)b * p.Hkv + g) * p.max_blocks + lb] = ok ? acc : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Top-K: radix select on order-preserving 64-bit keys, ties to the lower index
// ---------------------------------------------------------------------------

struct TopkParams {
  int* out;                // [B, H_kv, K]
  const double* scores;    // [B, H_kv, max_blocks]
  const int* ctx;
  int Hkv, bs, max_blocks, max_ctx, K;
};

__device__ __forceinline__ unsigned long long score_key(double x) {
  if (x == 0.0) x = 0.0;  // +0 and -0 are equal scores: give them one key
  const long long bits = __double_as_longlong(x);
  return bits < 0 ? ~(unsigned long long)bits : ((unsigned long long)bits | 0x8000000000000000ull);
}

// Exclusive prefix sum of v over the 256 threads; *total receives the sum.
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int x = s_wave[w];
    off += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

__global__ __launch_bounds__(256) void quest_topk_kernel(const TopkParams p) {
  __shared__ unsigned hist[256];
  __shared__ int s_wave[4];
  __shared__ int s_digit, s_above, s_cnt;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int n = (ctx + p.bs - 1) / p.bs;
  const int K = p.K;
  int* out = p.out + ((size_t)b * p.Hkv + g) * K;
  if (K >= n) {  // every block is selected
    for (int i = tid; i < K; i += 256) out[i] = i < n ? i : -1;
    return;
  }
  const double* sc = p.scores + ((size_t)b * p.Hkv + g) * p.max_blocks;
  const int C = (n + 255) / 256;
  const int i0 = min(n, tid * C), i1 = min(n, i0 + C);

  unsigned long long prefix = 0, mask = 0;
  int need = K, shift = 56;
  if (tid == 0) {
    s_digit = 0;
    s_above = 0;
    s_cnt = 0;
  }
  for (int pass = 0; pass < 8; ++pass) {
    shift = 56 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int i = i0; i < i1; ++i) {
      const unsigned long long key = score_key(sc[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending order of keys)
      unsigned c[4], t = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c[k] = hist[255 - 4 * tid - k];
        t += c[k];
      }
      unsigned inc = t;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned x = __shfl_up(inc, o);
        if (tid >= o) inc += x;
      }
      const unsigned excl = inc - t;
      if (excl < (unsigned)need && (unsigned)need <= inc) {
        unsigned above = excl;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (above + c[k] >= (unsigned)need) {
            s_digit = 255 - 4 * tid - k;
            s_above = (int)above;
            s_cnt = (int)c[k];
            break;
          }
          above += c[k];
        }
      }
    }
    __syncthreads();
    const int digit = s_digit, above = s_above, cnt = s_cnt;
    need -= above;
    prefix |= (unsigned long long)digit << shift;
    mask |= 0xFFull << shift;
    __syncthreads();
    if (cnt == need) break;  // the whole bucket is selected
  }

  // Selected: keys above the resolved prefix, plus the first `need` (by index)
  // of those equal to it.
  const unsigned long long ref = prefix >> shift;
  int n_eq = 0;
  for (int i = i0; i < i1; ++i) n_eq += (score_key(sc[i]) >> shift) == ref;
  int tot;
  int rank = block_exclusive_scan(n_eq, s_wave, &tot);
  int n_sel = 0;
  for (int i = i0; i < i1; ++i) {
    const unsigned long long k = score_key(sc[i]) >> shift;
    if (k > ref) {
      ++n_sel;
    } else if (k == ref) {
      n_sel += rank < need;
      ++rank;
    }
  }
  int pos = block_exclusive_scan(n_sel, s_wave, &tot);
  rank -= n_eq;
  for (int i = i0; i < i1; ++i) {
    const unsigned long long k = score_key(sc[i]) >> shift;
    bool sel = false;
    if (k > ref) {
      sel = true;
    } else if (k == ref) {
      sel = rank < need;
      ++rank;
    }
    if (sel && pos < K) out[pos++] = i;  // pos < K always holds; the check keeps writes in the row
  }
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
  int st = check_quest("quest_block_metadata", batch, num_kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len);
  if (st) return st;
  if (batch == 0 || max_context_len == 0) return GPKV_OK;
  if (!key_min || !key_max || !key_cache || !block_tables || !context_lens)
    return fail(GPKV_ERR_NULL, "quest_block_metadata: null pointer argument");
  MetaParams mp;
  mp.kmin = (unsigned short*)key_min;
  mp.kmax = (unsigned short*)key_max;
  mp.kc = (const unsigned char*)key_cache;
  mp.bt = block_tables;
  mp.ctx = context_lens;
  mp.NB = num_blocks;
  mp.row_bytes = num_kv_heads * head_dim * 2;
  mp.block_bytes = (long long)block_size * mp.row_bytes;
  mp.bs = block_size;
  mp.max_blocks = max_blocks_per_seq;
  mp.max_ctx = max_context_len;
  mp.last_only = last_block_only ? 1 : 0;
  const int max_nb = (max_context_len + block_size - 1) / block_size;
  const dim3 grid(last_block_only ? 1 : max_nb, batch);
  quest_meta_kernel<<<grid, dim3(256), 0, (hipStream_t)stream>>>(mp);
  return check_launch("quest_block_metadata");
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
  const char* fn = "quest_select_topk";
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
  if (max_nb > 0) {
    ScoreParams sp;
    sp.scores = (double*)workspace;
    sp.q = (const unsigned short*)query;
    sp.kmin = (const unsigned short*)key_min;
    sp.kmax = (const unsigned short*)key_max;
    sp.bt = block_tables;
    sp.ctx = context_lens;
    sp.NB = num_blocks;
    sp.Hq = num_q_heads;
    sp.Hkv = num_kv_heads;
    sp.G = num_q_heads / num_kv_heads;
    sp.bs = block_size;
    sp.max_blocks = max_blocks_per_seq;
    sp.max_ctx = max_context_len;
    const dim3 grid((max_nb + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG, num_kv_heads, batch);
    if (head_dim == 128)
      quest_score_kernel<128><<<grid, dim3(256), 0, s>>>(sp);
    else
      quest_score_kernel<64><<<grid, dim3(256), 0, s>>>(sp);
    st = check_launch(fn);
    if (st) return st;
  }
  TopkParams tp;
  tp.out = topk_indices;
  tp.scores = (const double*)workspace;
  tp.ctx = context_lens;
  tp.Hkv = num_kv_heads;
  tp.bs = block_size;
  tp.max_blocks = max_blocks_per_seq;
  tp.max_ctx = max_context_len;
  tp.K = topk_blocks;
  quest_topk_kernel<<<dim3(num_kv_heads, batch), dim3(256), 0, s>>>(tp);
  return check_launch(fn);
}
