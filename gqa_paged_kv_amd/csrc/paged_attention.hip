// GQA paged decode attention, dense and Quest-sparse: split-KV partials + combine.
//
// What is computed (["Ascend Kernel-to-Serving Pipeline", sections "GQA Paged
// Attention" and "Quest Sparse Attention"]): for each sequence b and query head h,
// softmax attention of q[b,h] over the tokens of b (all tokens < context_lens[b],
// or only those in the selected logical blocks), reading K/V of KV head
// h / G through block_tables, the ragged last block masked. The running max /
// normaliser / rescaled accumulator (online softmax) and the split + weighted
// combine ([TL18] = TileLang tutorial ch. 18, section 4.1) are how the kernels
// reach that result; they are not a different definition.
//
// Work decomposition (MI355X-first)
// ---------------------------------
// Workgroups hold 4 waves; the waves of a workgroup take different KV heads of
// the same tokens, so whole cache rows (every KV head of a token) stream from
// HBM together.
//  - Dense (balanced): the grid is one workgroup per compute unit. Each
//    workgroup computes the prefix sums of the sequences' 16-token sub-tile
//    counts (each plus a fixed cost for starting the sequence) and takes an
//    equal share of the flattened (sequence, sub-tile) space, so ragged batches
//    cost no tail: every workgroup moves about the same number of KV bytes, a
//    little less where it starts more sequences. A workgroup writes one partial
//    per sequence it touches into slot (workgroup + sequence), which is unique
//    because shares are ordered; the combine recomputes which workgroups covered
//    a sequence.
//  - Sparse, and dense batches too large for the balanced table: a workgroup per
//    (sequence, split of `split_tokens` virtual tokens), the split's block-table
//    entries (per KV head when sparse) staged in LDS.
//  - Decode append (the step's cache write in the same call, dense only): the split
//    phase stops one position short of each appending sequence's context, and the
//    combine merges that token from the call's inputs as one more unit and writes
//    it into the cache (after every read of the cache in the call).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "attention.h"

namespace gpkv {

// ---------------------------------------------------------------------------
// Split path: a workgroup per (sequence, split)
// ---------------------------------------------------------------------------

struct SplitParams {
  AttnCommon c;
  float* part_o;             // [B, H_kv, S, G, D] fp32
  float* part_lse;           // [B, H_kv, S, G] fp32 (base 2)
  const int* block_tables;   // [B, max_blocks]
  const int* ctx;            // [B]
  const int* topk;           // [B, H_kv, K] (sparse only)
  const long long* slots;    // decode append: [B] slot of each sequence's new token, or null
  long long NB;              // pool size; block ids outside [0, NB) select nothing
  int max_blocks, max_ctx, num_splits, split_tokens, topk_blocks;
};

template <int D, bool SPARSE, bool FP8>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(3))) void attn_split_kernel(const SplitParams p) {
  // Entry e covers virtual tokens [t0 + e*bs, t0 + (e+1)*bs): s_pb = physical
  // block (-1: nothing selected), s_tok0 = logical position of the block's row 0.
  // Dense: one table for all KV heads; sparse: one table per KV head.
  __shared__ int s_pb[kMaxTable];
  __shared__ int s_tok0[kMaxTable];

  const int split = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);  // tell the compiler the tile loop is wave-uniform
  const int bs = p.c.bs, Hkv = p.c.Hkv;
  const int ctx = split_ctx(p.ctx, p.slots, p.NB * bs, b, p.max_ctx);
  const int nb = (ctx + bs - 1) / bs;
  const int T = p.split_tokens;
  const int span = SPARSE ? p.topk_blocks * bs : ctx;
  const int t0 = split * T;
  if (t0 >= span) return;  // dense: past this sequence's context (the combine skips it)

  const int n_ent = T / bs;
  const int e0 = t0 / bs;
  const int n_tab = SPARSE ? Hkv * n_ent : n_ent;
  for (int i = tid; i < n_tab; i += blockDim.x) {
    const int e = SPARSE ? i % n_ent : i;
    const int ve = e0 + e;
    int lb;
    if (SPARSE) {
      const int gh = i / n_ent;
      lb = ve < p.topk_blocks ? p.topk[((size_t)b * Hkv + gh) * p.topk_blocks + ve] : -1;
    } else {
      lb = ve;
    }
    const int pb = (lb >= 0 && lb < nb) ? p.block_tables[(size_t)b * p.max_blocks + lb] : -1;
    const bool ok = pb >= 0 && pb < p.NB;
    s_pb[i] = ok ? pb : -1;
    s_tok0[i] = ok ? lb * bs : 0;
  }
  __syncthreads();

  const int G = p.c.G;
  for (int g = wave; g < Hkv; g += kWaves) {
    const int* tab_pb = s_pb + (SPARSE ? g * n_ent : 0);
    const int* tab_t0 = s_tok0 + (SPARSE ? g * n_ent : 0);
    auto desc = [&](int u, int& pb, int& row0, int& nv) {
      const int e = (16 * u) / bs;
      row0 = (16 * u) & (bs - 1);
      const int x = tab_pb[e];
      int n = ctx - (tab_t0[e] + row0);
      n = n < 0 ? 0 : (n > 16 ? 16 : n);
      if (x < 0) n = 0;
      nv = uniform(n);
      pb = uniform(x < 0 ? 0 : x);
    };
    const size_t unit = ((size_t)b * Hkv + g) * p.num_splits + split;
    const int rr = tid & 15;
    RowTiles<1> rows;
    rows.q[0] = rr < G ? p.c.q + ((size_t)b * p.c.Hq + (size_t)g * G + rr) * D : nullptr;
    rows.n_rows[0] = G;
    rows.limit[0] = 0;
    rows.o[0] = p.part_o + unit * G * D;
    rows.lse[0] = p.part_lse + unit * G;
    attend_head<D, FP8, false, 1>(p.c, g, T / 16, desc, 0, rows);
  }
}

// ---------------------------------------------------------------------------
// Balanced dense path: equal shares of the flattened (sequence, sub-tile) space
// ---------------------------------------------------------------------------

struct BalParams {
  AttnCommon c;
  float* part_o;             // [N + B, H_kv, G, D] fp32, slot = workgroup + sequence
  float* part_lse;           // [N + B, H_kv, G] fp32 (base 2)
  int* prefix;               // [B + 1] prefix sums of the sequences' costs (sub-tiles +
                             // kSegCost each), written by workgroup 0
  const int* block_tables;
  const int* ctx;
  const int* topk;           // [B, H_kv, K] logical block ids (sparse only)
  const long long* slots;    // decode append: [B] slot of each sequence's new token, or null
  long long NB;
  int B, max_blocks, max_ctx, nwg, topk_blocks;
};

// Cost of starting a sequence inside a share, in sub-tiles: each sequence's span of
// the flattened space opens with this many sub-tiles of no work, so shares that
// start many sequences (table staging, the first tile's loads, the partial row's
// write) take fewer sub-tiles. Measured (one workgroup per CU, 0 / 1 / 2 / 3 / 4 / 6):
// Qwen-shaped batch 59.1 / 58.0 / 57.4 / 57.6 / 57.5 / 57.7 us, 8K-average 173.8 /
// 172.5 / 172.2 / 172.2 / 172.4 / 173.2, ragged 8-KV-head batch 443 / 441 / 438 /
// 440 / 443 / 445; the 40960-token batch and the sparse calls did not move.
constexpr int kSegCost = 2;

// Work of a sequence, in 16-token sub-tiles: dense, its context; sparse,
// min(K, blocks) blocks. Valid ids of one KV head's list are distinct blocks of the
// sequence, so no head has more valid entries than that, wherever they sit in its
// list; lists from Top-K have exactly that many.
// Occupancy hint of two waves per SIMD (at most 256 registers), for this kernel and
// the direct sparse one: without it the compiler keeps the MFMA accumulators in AGPRs
// and copies them to VGPRs around every softmax (72 v_accvgpr moves per 32-token tile
// at D = 128, 242 VALU per tile against 170 with the hint).
template <int D, bool SPARSE, bool FP8, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_balanced_kernel(const BalParams p) {
  __shared__ int s_pref[kMaxBalBatch + 1];
  __shared__ int s_pb[kBalTab];                  // physical block per table entry (-1: none)
  __shared__ int s_tok0[SPARSE ? kBalTab : 1];   // sparse: logical position of its row 0
  __shared__ int s_wave[NW];
  const int wg = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int B = p.B, bs = p.c.bs, Hkv = p.c.Hkv, G = p.c.G;
  const int spb = bs >> 4;   // sub-tiles per block

  // Costs of every sequence (sub-tiles plus the start cost; an empty sequence costs
  // nothing), and their prefix sums (all workgroups compute the same values;
  // workgroup 0 also hands them to the combine).
  int carry = 0;
  for (int base = 0; base < B; base += NW * 64) {
    const int bb = base + tid;
    int n = 0;
    if (bb < B) {
      const int ctx = split_ctx(p.ctx, p.slots, p.NB * bs, bb, p.max_ctx);
      if (SPARSE) {
        const int nb = (ctx + bs - 1) / bs;
        n = (nb < p.topk_blocks ? nb : p.topk_blocks) * spb;
      } else {
        n = (ctx + 15) >> 4;
      }
    }
    n += n > 0 ? kSegCost : 0;
    int tot;
    const int ex = wg_exclusive_scan<NW>(n, s_wave, &tot);
    if (bb < B) s_pref[bb + 1] = carry + ex + n;
    carry += tot;
  }
  if (tid == 0) s_pref[0] = 0;
  __syncthreads();
  if (wg == 0)
    for (int i = tid; i <= B; i += NW * 64) p.prefix[i] = s_pref[i];
  const long long S = s_pref[B];
  const int s0 = (int)((long long)wg * S / p.nwg);
  const int s1 = (int)((long long)(wg + 1) * S / p.nwg);
  if (s0 >= s1) return;

  // First sequence of the share: the last b with prefix[b] <= s0.
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pref[mid] <= s0)
      lo = mid;
    else
      hi = mid - 1;
  }
  for (int b = lo; b < B && s_pref[b] < s1; ++b) {
    const int c0 = s_pref[b] + (s_pref[b + 1] > s_pref[b] ? kSegCost : 0);  // first sub-tile
    const int ub = (s0 > c0 ? s0 : c0) - c0;
    const int ue = (s1 < s_pref[b + 1] ? s1 : s_pref[b + 1]) - c0;
    if (ue <= ub) continue;  // empty sequence
    const int ctx = split_ctx(p.ctx, p.slots, p.NB * bs, b, p.max_ctx);
    const int nb = (ctx + bs - 1) / bs;
    // Table entries (blocks) the share touches: dense, logical blocks e0 ..;
    // sparse, positions e0 .. of each KV head's list with the invalid ids removed.
    const int e0 = ub / spb;
    const int n_ent = (ue - 1) / spb - e0 + 1;
    __syncthreads();  // the previous sequence's table is no longer read
    if (!SPARSE) {
      for (int e = tid; e < n_ent; e += NW * 64) {
        const int lb = e0 + e;
        const int pb = lb < nb ? p.block_tables[(size_t)b * p.max_blocks + lb] : -1;
        s_pb[e] = (pb >= 0 && pb < p.NB) ? pb : -1;
      }
    } else {
      for (int i = tid; i < Hkv * n_ent; i += NW * 64) s_pb[i] = -1;
      __syncthreads();
      // Compaction of each head's list, 64 entries per step: a valid entry's
      // position is the number of valid entries before it. Four steps' entries
      // are requested at once, so a share deep in a long list waits for one
      // round of list loads rather than one per 64 entries.
      constexpr int kListSteps = 4;
      for (int g = wave; g < Hkv; g += NW) {
        const int* lst = p.topk + ((size_t)b * Hkv + g) * p.topk_blocks;
        int run = 0;
        for (int c0 = 0; c0 < p.topk_blocks && run < e0 + n_ent; c0 += 64 * kListSteps) {
          int ids[kListSteps];
#pragma unroll
          for (int j = 0; j < kListSteps; ++j) {
            const int e = c0 + 64 * j + lane;
            ids[j] = e < p.topk_blocks ? lst[e] : -1;
          }
#pragma unroll
          for (int j = 0; j < kListSteps; ++j) {
            const int id = ids[j];
            const bool valid = id >= 0 && id < nb;
            const unsigned long long m = __ballot(valid);
            const int pos = run + __popcll(m & ((1ull << lane) - 1ull));
            if (valid && pos >= e0 && pos < e0 + n_ent) {
              const int pb = p.block_tables[(size_t)b * p.max_blocks + id];
              const int i = g * n_ent + (pos - e0);
              s_pb[i] = (pb >= 0 && pb < p.NB) ? pb : -1;
              s_tok0[i] = id * bs;
            }
            run += __popcll(m);
          }
        }
      }
    }
    __syncthreads();
    const size_t slot = (size_t)wg + b;
    for (int g = wave; g < Hkv; g += NW) {
      const int* tab = s_pb + (SPARSE ? g * n_ent : 0);
      const int* tok = s_tok0 + (SPARSE ? g * n_ent : 0);
      auto desc = [&](int u, int& pb, int& row0, int& nv) {
        const int v = ub + u;
        const int blk = v / spb;
        row0 = (v - blk * spb) * 16;
        const int x = tab[blk - e0];
        const int t0 = SPARSE ? tok[blk - e0] + row0 : 16 * v;
        int n = ctx - t0;
        n = n < 0 ? 0 : (n > 16 ? 16 : n);
        if (x < 0) n = 0;
        nv = uniform(n);
        pb = uniform(x < 0 ? 0 : x);
      };
      const size_t unit = slot * Hkv + g;
      const int rr = tid & 15;
      RowTiles<1> rows;
      rows.q[0] = rr < G ? p.c.q + ((size_t)b * p.c.Hq + (size_t)g * G + rr) * D : nullptr;
      rows.n_rows[0] = G;
      rows.limit[0] = 0;
      rows.o[0] = p.part_o + unit * G * D;
      rows.lse[0] = p.part_lse + unit * G;
      attend_head<D, FP8, false, 1>(p.c, g, ue - ub, desc, 0, rows);
    }
  }
}

// ---------------------------------------------------------------------------
// Direct sparse path: one workgroup per (sequence, KV head)
// ---------------------------------------------------------------------------

// Quest selects the same number of blocks, min(K, blocks), for every KV head of a
// sequence, so when the batch's (sequence, KV head) pairs fill the GPU one
// workgroup per pair is balanced without a global schedule. Its waves split the
// pair's selected sub-tiles, and their partial rows meet in LDS: the output is
// written here, with no partial rows in memory and no combine launch.
struct DirectParams {
  AttnCommon c;
  float* out;                // [B, H_q, D] fp32
  const int* block_tables;
  const int* ctx;
  const int* topk;           // [B, H_kv, K] logical block ids
  long long NB;
  int B, max_blocks, max_ctx, topk_blocks;
};

template <int D, bool FP8>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_sparse_direct_kernel(const DirectParams p) {
  __shared__ int s_pb[kDirTab];    // compacted list: physical block (-1: none)
  __shared__ int s_tok0[kDirTab];  // logical position of the block's row 0
  __shared__ __align__(16) float s_o[kWaves * kMaxGroup * D];
  __shared__ float s_lse[kWaves * kMaxGroup];
  __shared__ int s_wave[kWaves];
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int Hkv = p.c.Hkv, G = p.c.G, bs = p.c.bs, K = p.topk_blocks;
  const int b = blockIdx.x / Hkv, g = blockIdx.x - b * Hkv;
  const int ctx = clamp_ctx(p.ctx[b], p.max_ctx);
  const int nb = (ctx + bs - 1) / bs;
  const int spb = bs >> 4;

  // Compaction of the head's list: each thread takes a contiguous run of entries,
  // and a valid entry's position is the number of valid entries before it.
  const int* lst = p.topk + ((size_t)b * Hkv + g) * K;
  const int per = (K + kWaves * 64 - 1) / (kWaves * 64);
  const int e_begin = tid * per;
  int n_mine = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e_begin + i;
    const int id = e < K ? lst[e] : -1;
    n_mine += (id >= 0 && id < nb) ? 1 : 0;
  }
  int n_valid;
  int pos = wg_exclusive_scan(n_mine, s_wave, &n_valid);
  for (int i = 0; i < per && n_mine > 0; ++i) {
    const int e = e_begin + i;
    const int id = e < K ? lst[e] : -1;
    if (id >= 0 && id < nb) {
      const int pb = p.block_tables[(size_t)b * p.max_blocks + id];
      s_pb[pos] = (pb >= 0 && pb < p.NB) ? pb : -1;
      s_tok0[pos] = id * bs;
      ++pos;
    }
  }
  __syncthreads();

  // Wave w takes a contiguous quarter of the 32-token tiles.
  const int n_sub = n_valid * spb;
  const int n_tiles = (n_sub + 1) >> 1;
  const int ta = wave * n_tiles / kWaves, tb = (wave + 1) * n_tiles / kWaves;
  const int ub = 2 * ta;
  const int ue = 2 * tb < n_sub ? 2 * tb : n_sub;
  auto desc = [&](int u, int& pb, int& row0, int& nv) {
    const int v = ub + u;
    const int blk = v / spb;
    row0 = (v - blk * spb) * 16;
    const int x = s_pb[blk];
    int n = ctx - (s_tok0[blk] + row0);
    n = n < 0 ? 0 : (n > 16 ? 16 : n);
    if (x < 0) n = 0;
    nv = uniform(n);
    pb = uniform(x < 0 ? 0 : x);
  };
  const int rr = tid & 15;
  RowTiles<1> rows;
  rows.q[0] = rr < G ? p.c.q + ((size_t)b * p.c.Hq + (size_t)g * G + rr) * D : nullptr;
  rows.n_rows[0] = G;
  rows.limit[0] = 0;
  rows.o[0] = s_o + wave * kMaxGroup * D;
  rows.lse[0] = s_lse + wave * kMaxGroup;
  attend_head<D, FP8, false, 1>(p.c, g, ue > ub ? ue - ub : 0, desc, 0, rows);
  __syncthreads();

  // out = sum_w 2^(lse_w - M) O_w / sum_w 2^(lse_w - M); no valid token: zeros.
  float* dst = p.out + ((size_t)b * p.c.Hq + (size_t)g * G) * D;
  for (int i = tid; i < G * (D / 4); i += kWaves * 64) {
    const int h = i / (D / 4), d = 4 * (i - h * (D / 4));
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, s_lse[w * kMaxGroup + h]);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = __builtin_amdgcn_exp2f(s_lse[w * kMaxGroup + h] - m);
        acc += wt * *(const f32x4*)(s_o + (w * kMaxGroup + h) * D + d);
        den += wt;
      }
      acc *= 1.f / den;
    }
    *(f32x4*)(dst + (size_t)h * D + d) = acc;
  }
}

// ---------------------------------------------------------------------------
// Combine: out = sum_u w_u O_u / sum_u w_u, w_u = 2^(lse_u - max lse)
// ---------------------------------------------------------------------------

// Each unit's normaliser is taken relative to one common maximum ([TL18] 4.1).
// One 256-thread workgroup per (sequence, query head): 16-byte loads, D/4 threads
// per unit row, so a pass over the workgroup reads 256*4/D units at once and many
// unit rows are in flight.
struct CombineParams {
  float* out;               // [B, H_q, D]
  const float* part_o;
  const float* part_lse;
  const int* ctx;
  const int* prefix;        // balanced path
  int Hq, Hkv, G, max_ctx, num_splits, split_tokens, sparse, balanced, B, nwg;
  // Decode append (slots non-null): sequence b's new token (row b of knew / vnew)
  // joins the merge as one more unit, and the combine writes it into the cache at
  // its slot (and folds it into the Quest key min / max when kmin is non-null).
  const long long* slots;      // [B]
  long long num_slots;         // NB * bs
  const unsigned short* q;     // [B, H_q, D] bf16
  const unsigned short* knew;  // [B, H_kv, D] bf16
  const unsigned short* vnew;
  unsigned short* kc;          // [NB, bs, H_kv, D] bf16
  unsigned short* vc;
  unsigned short* kmin;        // [NB, H_kv, D] bf16, or null
  unsigned short* kmax;
  const float* k_scale;        // E4M3 caches: [H_kv] (codes = e4m3(x / scale))
  const float* v_scale;
  int bs;
  float qk_scale_log2;
};

// Four bf16 values (channels in order) as the E4M3 codes of x * inv, one byte each
// (the FP8 write path's quantisation).
__device__ __forceinline__ unsigned e4m3_codes4(uint2 x, float inv) {
  return e4m3_from_f32(bf16_lo(x.x) * inv) | (e4m3_from_f32(bf16_hi(x.x) * inv) << 8) |
         (e4m3_from_f32(bf16_lo(x.y) * inv) << 16) | (e4m3_from_f32(bf16_hi(x.y) * inv) << 24);
}

// Which new-token merge a combine instance does.
enum AppendMode { kNoAppend = 0, kAppendBf16 = 1, kAppendFp8 = 2 };

// Decode append: the new token's unit for query head g G + hl of sequence b, as
// thread c4 of the D / 4 threads holding the row's float4 columns sees it: base-2
// lse q . k_new * scale * log2(e) (the exact products summed in float32 over those
// threads, consecutive lanes of one wave that all call this) and the token's values.
// E4M3 caches: k_new and v_new are the values the cache will hold, code * scale of
// the codes the write stores.
template <int D, int MODE>
__device__ __forceinline__ void append_unit(const CombineParams& p, int b, int g, int hl, int c4,
                                            float& lse, f32x4& v) {
  constexpr int TPU = D / 4;
  const uint2 qq = *(const uint2*)(p.q + ((size_t)b * p.Hq + (size_t)g * p.G + hl) * D + 4 * c4);
  const size_t row = ((size_t)b * p.Hkv + g) * D + 4 * c4;
  uint2 kk = *(const uint2*)(p.knew + row);
  uint2 vv = *(const uint2*)(p.vnew + row);
  float kf = 1.f, vf = 1.f;
  if constexpr (MODE == kAppendFp8) {
    const float ks = p.k_scale[g], vs = p.v_scale[g];
    const float kinv = 1.0f / ks, vinv = 1.0f / vs;
    const u32x2 kd = e4m3x4_to_bf16(e4m3_codes4(kk, kinv));
    const u32x2 vd = e4m3x4_to_bf16(e4m3_codes4(vv, vinv));
    kk = uint2{kd[0], kd[1]};
    vv = uint2{vd[0], vd[1]};
    kf = ks;
    vf = vs;
  }
  float dot = bf16_lo(qq.x) * bf16_lo(kk.x);
  dot = __builtin_fmaf(bf16_hi(qq.x), bf16_hi(kk.x), dot);
  dot = __builtin_fmaf(bf16_lo(qq.y), bf16_lo(kk.y), dot);
  dot = __builtin_fmaf(bf16_hi(qq.y), bf16_hi(kk.y), dot);
#pragma unroll
  for (int o = TPU / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
  lse = dot * (p.qk_scale_log2 * kf);   // the split kernels' scale for this KV head
  v = f32x4{bf16_lo(vv.x), bf16_hi(vv.x), bf16_lo(vv.y), bf16_hi(vv.y)} * vf;
}

// Decode append: KV head g's part of sequence b's new token written into the cache at
// its slot (a slot outside the pool writes nothing, as the write path), with the
// Quest fold when the metadata is given; E4M3 caches take its codes. Threads t of nt
// share the row.
template <int D, int MODE>
__device__ __forceinline__ void append_write(const CombineParams& p, int b, int g, int t, int nt) {
  const long long s = p.slots[b];
  if (s < 0 || s >= p.num_slots) return;
  if constexpr (MODE == kAppendFp8) {
    // four channels per thread (D / 4 threads), so that the integer-arithmetic
    // encoding of the row's codes is spread wide
    const float kinv = 1.0f / p.k_scale[g], vinv = 1.0f / p.v_scale[g];
    const size_t src = ((size_t)b * p.Hkv + g) * D;
    const size_t dst = ((size_t)s * p.Hkv + g) * D;   // bytes
    for (int c = t; c < D / 4; c += nt) {
      const uint2 kk = *(const uint2*)(p.knew + src + 4 * c);
      const uint2 vv = *(const uint2*)(p.vnew + src + 4 * c);
      *(unsigned*)((unsigned char*)p.kc + dst + 4 * c) = e4m3_codes4(kk, kinv);
      *(unsigned*)((unsigned char*)p.vc + dst + 4 * c) = e4m3_codes4(vv, vinv);
    }
  } else {
    store_new_token<D>(p.knew, p.vnew, p.kc, p.vc, p.kmin, p.kmax, s, p.bs, p.Hkv, b, g, t, nt);
  }
}


// Units of (sequence b, KV head g, query head hl of the group) are u in
// [u_begin, u_end); unit u's lse and output sit at lse0 + u * lstride and
// o0 + u * ostride (balanced: u is a workgroup id and the slot is u + b).
struct UnitRange {
  int u_begin, u_end;
  long long S;
  bool check_live;          // only when some workgroups had an empty share
  const float* lse0;
  const float* o0;
  size_t lstride, ostride;
  int nwg;
  __device__ bool live(int u) const {
    if (!check_live) return true;
    return (long long)u * S / nwg < (long long)(u + 1) * S / nwg;
  }
};

template <int D>
__device__ __forceinline__ UnitRange unit_range(const CombineParams& p, int b, int g, int hl) {
  UnitRange r;
  const int G = p.G;
  r.nwg = p.nwg;
  r.S = 0;
  if (p.balanced) {
    long long pre0 = p.prefix[b];
    const long long pre1 = p.prefix[b + 1];
    r.S = p.prefix[p.B];
    if (pre1 <= pre0) {
      r.u_begin = r.u_end = 0;
    } else {
      pre0 += kSegCost;  // the sequence's first sub-tile
      r.u_begin = (int)(((pre0 + 1) * p.nwg - 1) / r.S);  // workgroup holding sub-tile pre0
      r.u_end = (int)((pre1 * p.nwg - 1) / r.S) + 1;      // ... and sub-tile pre1 - 1
    }
    r.lstride = (size_t)p.Hkv * G;
    r.ostride = r.lstride * D;
    r.lse0 = p.part_lse + ((size_t)b * p.Hkv + g) * G + hl;
    r.o0 = p.part_o + (((size_t)b * p.Hkv + g) * G + hl) * D;
  } else {
    const int ctx = split_ctx(p.ctx, p.slots, p.num_slots, b, p.max_ctx);
    r.u_begin = 0;
    r.u_end = p.sparse ? p.num_splits : (ctx + p.split_tokens - 1) / p.split_tokens;
    const size_t unit0 = ((size_t)b * p.Hkv + g) * p.num_splits;
    r.lstride = G;
    r.ostride = (size_t)G * D;
    r.lse0 = p.part_lse + unit0 * G + hl;
    r.o0 = p.part_o + (unit0 * G + hl) * D;
  }
  r.check_live = p.balanced && r.S < p.nwg;
  return r;
}

// Few units per sequence: one workgroup per (sequence, KV head); each group of
// D/4 threads (a "slot") owns query heads hl, hl + slots, ... of the group and
// merges that head's units on its own, without barriers: up to kHeadUnits unit
// rows in one round of loads after the prefix. In the append calls no merging wave
// writes the new token (its merge would wait for the write's loads): when the grid stays
// resident with one more wave per workgroup (WRITER 1), that wave writes KV head g's
// part; otherwise (WRITER 2) workgroup H_kv of each sequence writes every KV head's
// part. 8K-average batch (WRITER 1 against the first wave writing): the call 171.9 ->
// 171.2 us (bf16, with the Quest fold), 96.4 -> 95.4 us (E4M3); a fifth wave on the
// ragged 8-KV-head batch's eight workgroups per CU cost a second round of them
// (443 -> 449 us), hence WRITER 2 there (against the first wave writing: 439.4 ->
// 437.9 us bf16, 250.9 -> 248.9 us E4M3, medians of four runs).
constexpr int kHeadUnits = 12;

template <int D, int MODE, int WRITER, int NU>
__global__ __launch_bounds__(kCombineThreads + (WRITER == 1 ? 64 : 0)) void attn_combine_heads_kernel(const CombineParams p) {
  constexpr int TPU = D / 4;
  constexpr int SLOTS = kCombineThreads / TPU;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int slot = tid / TPU, c4 = tid % TPU;
  constexpr bool APPEND = MODE != kNoAppend;
  static_assert(APPEND == (WRITER != 0), "the append instances have a writer");
  if constexpr (WRITER == 1) {
    if (tid >= kCombineThreads) {
      append_write<D, MODE>(p, b, g, tid - kCombineThreads, 64);
      return;
    }
  } else if constexpr (WRITER == 2) {
    if (g == p.Hkv) {
      constexpr int PER = MODE == kAppendFp8 ? D / 4 : D / 8;   // threads per KV head's row
      for (int gg = tid / PER; gg < p.Hkv; gg += kCombineThreads / PER)
        append_write<D, MODE>(p, b, gg, tid % PER, PER);
      return;
    }
  }
  const bool append = APPEND && append_token(p.slots, p.num_slots, b, p.ctx, p.max_ctx);
  for (int hl = slot; hl < p.G; hl += SLOTS) {
    const UnitRange r = unit_range<D>(p, b, g, hl);
    const int u0 = r.u_begin;
    MergeState st = merge_rows_state<NU>(
        r.u_end - u0, r.lse0 + (size_t)u0 * r.lstride, r.lstride,
        r.o0 + (size_t)u0 * r.ostride + 4 * c4, r.ostride, [&](int k) { return r.live(u0 + k); });
    if (append) {
      float l;
      f32x4 v;
      append_unit<D, MODE>(p, b, g, hl, c4, l, v);
      merge_one(st, l, v);
    }
    *(f32x4*)(p.out + ((size_t)b * p.Hq + (size_t)g * p.G + hl) * D + 4 * c4) = merge_finish(st);
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(const CombineParams p) {
  constexpr int TPU = D / 4;                       // threads per unit row
  constexpr int UPP = kCombineThreads / TPU;       // units per pass
  __shared__ float s_red[kCombineThreads];
  __shared__ f32x4 s_acc[UPP][TPU];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  constexpr bool APPEND = MODE != kNoAppend;
  if constexpr (APPEND) {
    // Workgroups Hq + g of the append instances write KV head g's part of the new
    // token, so no merging workgroup waits for the write's loads (Qwen-shaped batch,
    // medians of four runs: bf16 with the Quest fold 59.0 -> 58.4 us, E4M3 39.0 -> 38.2).
    if (h >= p.Hq) {
      append_write<D, MODE>(p, b, h - p.Hq, tid, kCombineThreads);
      return;
    }
  }
  const int G = p.G;
  const int g = h / G, hl = h - g * G;
  float* out = p.out + ((size_t)b * p.Hq + h) * D;

  const bool append = APPEND && append_token(p.slots, p.num_slots, b, p.ctx, p.max_ctx);
  const UnitRange r = unit_range<D>(p, b, g, hl);
  if (r.u_end <= r.u_begin) {   // no unit: the appended token alone, or nothing
    if (tid < TPU) {
      MergeState st{f32x4{0.f, 0.f, 0.f, 0.f}, 0.f, -INFINITY};
      if (append) {
        float l;
        f32x4 v;
        append_unit<D, MODE>(p, b, g, hl, tid, l, v);
        merge_one(st, l, v);
      }
      *(f32x4*)(out + 4 * tid) = merge_finish(st);
    }
    return;
  }
  const int u_begin = r.u_begin, u_end = r.u_end;
  const float* lse0 = r.lse0;
  const float* o0 = r.o0;
  const size_t lstride = r.lstride, ostride = r.ostride;
  auto live = [&](int u) { return r.live(u); };

  // Thread (unit slot us, float4 column c4) walks units us, us+UPP, ..., eight
  // unit rows (lse and output) requested at once, and keeps its sum relative to
  // the largest lse it has seen (mr, -inf while it has seen only empty units); the
  // slots then meet in LDS under their common maximum. With up to 8*UPP units this
  // is one round of loads after the prefix.
  constexpr int UNROLL = 8;
  const int us = tid / TPU, c4 = tid % TPU;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f, mr = -INFINITY;
  for (int u = u_begin + us; u < u_end; u += UNROLL * UPP) {
    float l[UNROLL];
    f32x4 v[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const int uu = u + k * UPP;
      const bool ok = uu < u_end && live(uu);
      l[k] = ok ? lse0[(size_t)uu * lstride] : -INFINITY;
      v[k] = ok ? *(const f32x4*)(o0 + (size_t)uu * ostride + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m = mr;
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) m = fmaxf(m, l[k]);
    if (m == -INFINITY) continue;           // nothing valid yet
    const float s = __builtin_amdgcn_exp2f(mr - m);   // 0 when mr = -inf
    W *= s;
    acc *= s;
    mr = m;
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const float w = __builtin_amdgcn_exp2f(l[k] - m);
      W += w;
      acc += w * v[k];
    }
  }
  s_acc[us][c4] = acc;
  if (c4 == 0) {
    s_red[us] = W;
    s_red[UPP + us] = mr;
  }
  __syncthreads();
  if (tid < TPU) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < UPP; ++k) M = fmaxf(M, s_red[UPP + k]);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    float wt = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < UPP; ++k) {
        const float sk = __builtin_amdgcn_exp2f(s_red[UPP + k] - M);   // 0 for empty slots
        a += sk * s_acc[k][tid];
        wt += sk * s_red[k];
      }
    }
    MergeState st{a, wt, M};
    if (append) {
      float l;
      f32x4 v;
      append_unit<D, MODE>(p, b, g, hl, tid, l, v);
      merge_one(st, l, v);
    }
    *(f32x4*)(out + 4 * tid) = merge_finish(st);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups of the balanced kernel: one per compute unit. Measured on MI355X
// over an 8K-average ragged batch: one 4-wave workgroup per CU streams the KV
// cache at ~6.1 TB/s, while two or three per CU (all resident) reach only 5.7
// and 5.4 TB/s, and counts that are not a multiple of the CU count (192, 320,
// 384) leave some CUs with two shares. One wave per SIMD, each with a 32-token
// tile in flight, already covers HBM latency; more concurrent streams only add
// DRAM conflicts.
int balanced_capacity() {
  static std::mutex mu;
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  int& slot = cache[dev];
  if (slot == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
      (void)hipGetLastError();
      return 256;
    }
    slot = cus;
  }
  return slot;
}

struct Plan {
  bool balanced, direct;
  int split_tokens, num_splits, nwg;
  size_t o_bytes, lse_bytes, prefix_bytes;
};

// GPKV_ATTN_SCHEDULE=balanced|split|direct forces the schedule (tuning and test
// switch, read per call; direct applies to sparse calls only); by default the
// balanced schedule serves every batch its prefix and tables fit. The workspace
// size does not depend on the choice.
static Plan make_plan(bool sparse, int B, int Hq, int Hkv, int D, int bs, int span) {
  Plan pl;
  const int G = Hq / Hkv;
  const int spb = bs / 16;
  pl.balanced = B <= kMaxBalBatch && (!sparse || kBalTab / Hkv >= 3);
  // Sparse: the direct path when the (sequence, KV head) pairs fill the GPU and are
  // all resident at once (two workgroups per CU). With more pairs each later round
  // of workgroups pays the list -> table -> first tile latency again: 2048 pairs of
  // ragged sequences ran 18% slower than the balanced schedule and its combine.
  const bool direct_fits = sparse && span / bs <= kDirTab && (long long)B * Hkv <= (1LL << 22);
  const long long pairs = (long long)B * Hkv;
  pl.direct = direct_fits && pairs >= balanced_capacity() && pairs <= 2LL * balanced_capacity();
  const char* forced = getenv("GPKV_ATTN_SCHEDULE");
  if (forced && strcmp(forced, "split") == 0) pl.balanced = pl.direct = false;
  if (forced && strcmp(forced, "balanced") == 0) pl.direct = false;
  if (forced && strcmp(forced, "direct") == 0) pl.direct = direct_fits;
  pl.split_tokens = split_tokens_for(B, Hkv, span);
  const int per_token_entries = sparse ? Hkv : 1;
  while (pl.split_tokens > 128 && (pl.split_tokens / bs) * per_token_entries > kMaxTable)
    pl.split_tokens >>= 1;
  pl.num_splits = (span + pl.split_tokens - 1) / pl.split_tokens;
  if (pl.num_splits < 1) pl.num_splits = 1;
  size_t units;
  if (pl.balanced) {
    // One workgroup per CU, more only if a share would exceed the per-workgroup
    // table (sparse: H_kv entries per block of the share); never more than there
    // are sub-tiles.
    const long long max_sub = sparse ? (long long)B * (span / bs) * spb : (long long)B * ((span + 15) / 16);
    const long long share_max = sparse ? (long long)(kBalTab / Hkv - 2) * spb : kMaxSubPerWG;
    const long long max_cost = max_sub + (long long)B * kSegCost;
    long long n = balanced_capacity();
    const long long need = (max_cost + share_max - 1) / share_max;
    if (n < need) n = need;
    if (n > max_sub) n = max_sub;
    if (n < 1) n = 1;
    pl.nwg = (int)n;
    units = ((size_t)pl.nwg + B) * Hkv;
  } else {
    pl.nwg = 0;
    units = (size_t)B * Hkv * pl.num_splits;
  }
  pl.o_bytes = align256(units * G * D * sizeof(float));
  pl.lse_bytes = align256(units * G * sizeof(float));
  pl.prefix_bytes = pl.balanced ? align256(((size_t)B + 1) * sizeof(int)) : 0;
  return pl;
}

int check_common(const char* fn, int B, int Hq, int Hkv, int D, int bs, long long NB,
                        int max_blocks, int max_ctx) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || NB < 0 || max_blocks <= 0 || max_ctx < 0)
    return fail(GPKV_ERR_SHAPE,
                "%s: batch=%d num_q_heads=%d num_kv_heads=%d num_blocks=%lld "
                "max_blocks_per_seq=%d max_context_len=%d",
                fn, B, Hq, Hkv, NB, max_blocks, max_ctx);
  if (Hq % Hkv != 0)
    return fail(GPKV_ERR_SHAPE, "%s: num_q_heads=%d is not a multiple of num_kv_heads=%d", fn,
                Hq, Hkv);
  if (Hq / Hkv > kMaxGroup)
    return fail(GPKV_ERR_UNSUPPORTED, "%s: group size %d > %d", fn, Hq / Hkv, kMaxGroup);
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

// Many units per sequence (per_head): one workgroup per query head, its threads spread
// over the units. Few units: one workgroup per KV head, a slot of threads per query head.
template <int D, int MODE>
static void launch_combine_mode(bool per_head, bool few_units, int B, int Hq, int Hkv,
                                hipStream_t stream, const CombineParams& cp) {
  const dim3 cblock(kCombineThreads), grid(Hkv, B);
  const bool write_wave = (long long)B * Hkv <= 4LL * balanced_capacity();
  // Unit rows requested at once: kHeadUnits (eight in the append instances, so that the
  // new token's unit fits four waves per SIMD), or four when sequences hold few units:
  // 53-60 registers instead of 96-125, eight waves per SIMD instead of four or five, so
  // that a grid of eight workgroups per CU is resident at once. Ragged 8-KV-head batch
  // (2048 workgroups, medians of four runs): dense 440.0 -> 436.1 us, sparse 347.3 ->
  // 342.7, E4M3 dense 244.5 -> 241.4, dense append 440.9 -> 439.3.
  constexpr int NU = MODE != kNoAppend ? 8 : kHeadUnits;
  if (per_head) {   // + one write workgroup per KV head in the append instances
    attn_combine_kernel<D, MODE><<<dim3(Hq + (MODE != kNoAppend ? Hkv : 0), B), cblock, 0, stream>>>(cp);
  } else if constexpr (MODE == kNoAppend) {
    if (few_units)
      attn_combine_heads_kernel<D, MODE, 0, 4><<<grid, cblock, 0, stream>>>(cp);
    else
      attn_combine_heads_kernel<D, MODE, 0, NU><<<grid, cblock, 0, stream>>>(cp);
  } else if (write_wave) {
    attn_combine_heads_kernel<D, MODE, 1, NU><<<grid, dim3(kCombineThreads + 64), 0, stream>>>(cp);
  } else {
    const dim3 wgrid(Hkv + 1, B);   // + the writing workgroup of each sequence
    if (few_units)
      attn_combine_heads_kernel<D, MODE, 2, 4><<<wgrid, cblock, 0, stream>>>(cp);
    else
      attn_combine_heads_kernel<D, MODE, 2, NU><<<wgrid, cblock, 0, stream>>>(cp);
  }
}

template <int D>
static void launch_combine(bool per_head, bool few_units, int mode, int B, int Hq, int Hkv,
                           hipStream_t stream, const CombineParams& cp) {
  if (mode == kAppendFp8)
    launch_combine_mode<D, kAppendFp8>(per_head, few_units, B, Hq, Hkv, stream, cp);
  else if (mode == kAppendBf16)
    launch_combine_mode<D, kAppendBf16>(per_head, few_units, B, Hq, Hkv, stream, cp);
  else
    launch_combine_mode<D, kNoAppend>(per_head, few_units, B, Hq, Hkv, stream, cp);
}

// GPKV_BAL_WIDE=0 keeps four waves per balanced workgroup everywhere (tuning and test
// switch, read per call).
static bool getenv_wide() {
  const char* f = getenv("GPKV_BAL_WIDE");
  return !(f && strcmp(f, "0") == 0);
}

template <int D, bool SPARSE, bool FP8>
static void launch_attention(bool balanced, const BalParams& bp, const SplitParams& sp, int nwg,
                             int num_splits, int B, hipStream_t stream) {
  const dim3 block(kWaves * 64);
  // 8 KV heads or a multiple: eight waves per workgroup (one per KV head of the share's
  // tokens, two per SIMD). Measured on MI355X over the ragged 8-KV-head batch, outputs
  // bit-identical: dense over E4M3 caches 256-263 -> 250 us (one wave's code decoding
  // overlaps the other's loads), over bf16 unchanged (441-445 us); sparse over E4M3
  // 206-212 -> 197-198 us, over bf16 351-353 -> 345-348 us.
  if (balanced && bp.c.Hkv % 8 == 0 && getenv_wide())
    attn_balanced_kernel<D, SPARSE, FP8, 8><<<dim3(nwg), dim3(8 * 64), 0, stream>>>(bp);
  else if (balanced)
    attn_balanced_kernel<D, SPARSE, FP8, kWaves><<<dim3(nwg), block, 0, stream>>>(bp);
  else
    attn_split_kernel<D, SPARSE, FP8><<<dim3(num_splits, B), block, 0, stream>>>(sp);
}

// Decode append inputs (gpkv_paged_attention_decode_append): the new tokens' rows,
// their slots and the Quest metadata to fold them into (null: none).
struct AppendArgs {
  const void* key;
  const void* value;
  void* key_min;
  void* key_max;
  const int64_t* slots;
};

static int attn_run(bool sparse, bool fp8, float* out, const void* query, const void* kc,
                    const void* vc, const float* k_scale, const float* v_scale, const int* bt,
                    const int* ctx, const int* topk, int B, int Hq, int Hkv, int D, int bs,
                    long long NB, int max_blocks, int max_ctx, int K, float scale, void* ws,
                    size_t ws_bytes, hipStream_t stream, const AppendArgs* app = nullptr) {
  const char* fn = app ? (fp8 ? "paged_attention_decode_fp8_append" : "paged_attention_decode_append")
                : sparse ? (fp8 ? "sparse_paged_attention_decode_fp8" : "sparse_paged_attention_decode")
                         : (fp8 ? "paged_attention_decode_fp8" : "paged_attention_decode");
  int st = check_common(fn, B, Hq, Hkv, D, bs, NB, max_blocks, max_ctx);
  if (st) return st;
  if (sparse && K < 1) return fail(GPKV_ERR_SHAPE, "%s: topk_blocks=%d < 1", fn, K);
  if (B == 0) return GPKV_OK;
  if (!out || !query || !kc || !vc || !bt || !ctx || (sparse && !topk) ||
      (fp8 && (!k_scale || !v_scale)) ||
      (app && (!app->key || !app->value || !app->slots || (!app->key_min != !app->key_max))))
    return fail(GPKV_ERR_NULL, "%s: null pointer argument", fn);
  const long long span_ll = sparse ? (long long)K * bs : (long long)max_ctx;
  if (span_ll > (1LL << 30)) return fail(GPKV_ERR_SHAPE, "%s: token span too large", fn);
  if (sparse && (128 / bs) * Hkv > kMaxTable)
    return fail(GPKV_ERR_UNSUPPORTED, "%s: num_kv_heads=%d too large for block_size %d", fn, Hkv,
                bs);
  const Plan pl = make_plan(sparse, B, Hq, Hkv, D, bs, (int)span_ll);
  const size_t need = pl.o_bytes + pl.lse_bytes + pl.prefix_bytes;
  if (!ws || ws_bytes < need)
    return fail(GPKV_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn,
                ws ? ws_bytes : (size_t)0, need);

  const int G = Hq / Hkv;
  AttnCommon c;
  c.q = (const unsigned short*)query;
  c.kc = (const unsigned char*)kc;
  c.vc = (const unsigned char*)vc;
  c.k_scale = k_scale;
  c.v_scale = v_scale;
  c.row_bytes = Hkv * D * (fp8 ? 1 : 2);
  c.block_bytes = (long long)bs * c.row_bytes;
  c.Hq = Hq;
  c.Hkv = Hkv;
  c.G = G;
  c.bs = bs;
  c.qk_scale_log2 = scale * 1.4426950408889634f;
  float* part_o = (float*)ws;
  float* part_lse = (float*)((char*)ws + pl.o_bytes);
  int* prefix = (int*)((char*)ws + pl.o_bytes + pl.lse_bytes);

  if (pl.direct) {
    DirectParams dp;
    dp.c = c;
    dp.out = out;
    dp.block_tables = bt;
    dp.ctx = ctx;
    dp.topk = topk;
    dp.NB = NB;
    dp.B = B;
    dp.max_blocks = max_blocks;
    dp.max_ctx = max_ctx;
    dp.topk_blocks = K;
    const dim3 grid((unsigned)((long long)B * Hkv)), block(kWaves * 64);
    if (D == 128) {
      if (fp8)
        attn_sparse_direct_kernel<128, true><<<grid, block, 0, stream>>>(dp);
      else
        attn_sparse_direct_kernel<128, false><<<grid, block, 0, stream>>>(dp);
    } else {
      if (fp8)
        attn_sparse_direct_kernel<64, true><<<grid, block, 0, stream>>>(dp);
      else
        attn_sparse_direct_kernel<64, false><<<grid, block, 0, stream>>>(dp);
    }
    return check_launch(fn);
  }

  BalParams bp;
  bp.c = c;
  bp.part_o = part_o;
  bp.part_lse = part_lse;
  bp.prefix = prefix;
  bp.block_tables = bt;
  bp.ctx = ctx;
  bp.topk = topk;
  bp.slots = app ? (const long long*)app->slots : nullptr;
  bp.NB = NB;
  bp.B = B;
  bp.max_blocks = max_blocks;
  bp.max_ctx = max_ctx;
  bp.nwg = pl.nwg;
  bp.topk_blocks = sparse ? K : 0;
  SplitParams sp;
  sp.c = c;
  sp.part_o = part_o;
  sp.part_lse = part_lse;
  sp.block_tables = bt;
  sp.ctx = ctx;
  sp.topk = topk;
  sp.slots = bp.slots;
  sp.NB = NB;
  sp.max_blocks = max_blocks;
  sp.max_ctx = max_ctx;
  sp.num_splits = pl.num_splits;
  sp.split_tokens = pl.split_tokens;
  sp.topk_blocks = sparse ? K : 0;
  const int sel = (D == 128 ? 4 : 0) + (sparse ? 2 : 0) + (fp8 ? 1 : 0);
  switch (sel) {
    case 0: launch_attention<64, false, false>(pl.balanced, bp, sp, pl.nwg, pl.num_splits, B, stream); break;
    case 1: launch_attention<64, false, true>(pl.balanced, bp, sp, pl.nwg, pl.num_splits, B, stream); break;
    case 2: launch_attention<64, true, false>(pl.balanced, bp, sp, pl.nwg, pl.num_splits, B, stream); break;
    case 3: launch_attention<64, true, true>(pl.balanced, bp, sp, pl.nwg, pl.num_splits, B, stream); break;
    case 4: launch_attention<128, false, false>(pl.balanced, bp, sp, pl.nwg, pl.num_splits, B, stream); break;
    case 5: launch_attention<128, false, true>(pl.balanced, bp, sp, pl.nwg, pl.num_splits, B, stream); break;
    case 6: launch_attention<128, true, false>(pl.balanced, bp, sp, pl.nwg, pl.num_splits, B, stream); break;
    default: launch_attention<128, true, true>(pl.balanced, bp, sp, pl.nwg, pl.num_splits, B, stream); break;
  }
  st = check_launch(fn);
  if (st) return st;

  CombineParams cp;
  cp.out = out;
  cp.part_o = part_o;
  cp.part_lse = part_lse;
  cp.ctx = ctx;
  cp.prefix = prefix;
  cp.Hq = Hq;
  cp.Hkv = Hkv;
  cp.G = G;
  cp.max_ctx = max_ctx;
  cp.num_splits = pl.num_splits;
  cp.split_tokens = pl.split_tokens;
  cp.sparse = sparse ? 1 : 0;
  cp.balanced = pl.balanced ? 1 : 0;
  cp.B = B;
  cp.nwg = pl.nwg;
  cp.slots = bp.slots;
  cp.num_slots = NB * bs;
  cp.q = (const unsigned short*)query;
  cp.knew = app ? (const unsigned short*)app->key : nullptr;
  cp.vnew = app ? (const unsigned short*)app->value : nullptr;
  cp.kc = (unsigned short*)kc;   // written only by the append call, whose caches are writable
  cp.vc = (unsigned short*)vc;
  cp.kmin = app ? (unsigned short*)app->key_min : nullptr;
  cp.kmax = app ? (unsigned short*)app->key_max : nullptr;
  cp.k_scale = k_scale;
  cp.v_scale = v_scale;
  cp.bs = bs;
  cp.qk_scale_log2 = c.qk_scale_log2;
  // Many units per sequence (long sequences over many workgroups or splits): one
  // workgroup per query head, its threads spread over the units. Few units: one
  // workgroup per KV head, a slot of threads per query head.
  const long long units_per_seq = pl.balanced ? (long long)pl.nwg / B + 1 : pl.num_splits;
  // The append calls' combine is its own instance: its extra registers (the new
  // token's unit) stay out of the plain combine.
  const int mode = cp.slots == nullptr ? kNoAppend : (fp8 ? kAppendFp8 : kAppendBf16);
  if (D == 128)
    launch_combine<128>(units_per_seq >= 6, units_per_seq <= 3, mode, B, Hq, Hkv, stream, cp);
  else
    launch_combine<64>(units_per_seq >= 6, units_per_seq <= 3, mode, B, Hq, Hkv, stream, cp);
  return check_launch(fn);
}

}  // namespace gpkv

using namespace gpkv;

extern "C" size_t gpkv_paged_attention_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                       int32_t num_kv_heads, int32_t head_dim,
                                                       int32_t block_size,
                                                       int32_t max_context_len) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      !supported_head_dim(head_dim) || !supported_block_size(block_size) || max_context_len < 0)
    return 0;
  const Plan pl = make_plan(false, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                            max_context_len);
  return pl.o_bytes + pl.lse_bytes + pl.prefix_bytes;
}

extern "C" size_t gpkv_sparse_attention_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                        int32_t num_kv_heads, int32_t head_dim,
                                                        int32_t block_size, int32_t topk_blocks) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      !supported_head_dim(head_dim) || !supported_block_size(block_size) || topk_blocks < 1 ||
      (long long)topk_blocks * block_size > (1LL << 30))
    return 0;
  const Plan pl = make_plan(true, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                            topk_blocks * block_size);
  return pl.o_bytes + pl.lse_bytes + pl.prefix_bytes;
}

extern "C" int gpkv_paged_attention_decode(float* out, const void* query, const void* key_cache,
                                           const void* value_cache, const int32_t* block_tables,
                                           const int32_t* context_lens, int32_t batch,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int64_t num_blocks, int32_t max_blocks_per_seq,
                                           int32_t max_context_len, float scale, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  clear_error();
  return attn_run(false, false, out, query, key_cache, value_cache, nullptr, nullptr,
                  block_tables, context_lens, nullptr, batch, num_q_heads, num_kv_heads, head_dim,
                  block_size, num_blocks, max_blocks_per_seq, max_context_len, 0, scale,
                  workspace, workspace_bytes, (hipStream_t)stream);
}

extern "C" int gpkv_paged_attention_decode_append(
    float* out, const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, void* key_min, void* key_max, const int64_t* slot_mapping,
    const int32_t* block_tables, const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, void* workspace,
    size_t workspace_bytes, void* stream) {
  clear_error();
  AppendArgs app{key, value, key_min, key_max, slot_mapping};
  return attn_run(false, false, out, query, key_cache, value_cache, nullptr, nullptr,
                  block_tables, context_lens, nullptr, batch, num_q_heads, num_kv_heads, head_dim,
                  block_size, num_blocks, max_blocks_per_seq, max_context_len, 0, scale,
                  workspace, workspace_bytes, (hipStream_t)stream, &app);
}

extern "C" int gpkv_paged_attention_decode_fp8_append(
    float* out, const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, const float* k_scale, const float* v_scale, const int64_t* slot_mapping,
    const int32_t* block_tables, const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, float scale, void* workspace,
    size_t workspace_bytes, void* stream) {
  clear_error();
  AppendArgs app{key, value, nullptr, nullptr, slot_mapping};
  return attn_run(false, true, out, query, key_cache, value_cache, k_scale, v_scale,
                  block_tables, context_lens, nullptr, batch, num_q_heads, num_kv_heads, head_dim,
                  block_size, num_blocks, max_blocks_per_seq, max_context_len, 0, scale,
                  workspace, workspace_bytes, (hipStream_t)stream, &app);
}

// ---------------------------------------------------------------------------
// Dense decode without allocation: the workspace is a file-scope device array
// ---------------------------------------------------------------------------

// Each GPU the library runs on holds its own copy of this array from the first
// launch until the process ends. In host code `scratch` names a host-side stand-in,
// never the device copy: host code uses only the per-device address that
// scratch_address() looks up.
static __device__ __align__(256) unsigned char scratch[GPKV_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device: looked up with
// hipGetSymbolAddress on the first call on that device (with it current), then
// kept per device.
static int scratch_address(const char* fn, void** ptr) {
  static std::mutex mu;
  static void* addr[64];
  int dev = -1;
  const hipError_t ed = hipGetDevice(&dev);
  if (ed != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return fail(GPKV_ERR_HIP, "%s: no current HIP device (%s)", fn, hipGetErrorString(ed));
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(GPKV_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn,
                  dev, hipGetErrorString(e));
    }
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return GPKV_OK;
}

extern "C" int gpkv_paged_attention_decode_noalloc(float* out, const void* query,
                                                   const void* key_cache, const void* value_cache,
                                                   const int32_t* block_tables,
                                                   const int32_t* context_lens, int32_t batch,
                                                   int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_dim, int32_t block_size,
                                                   int64_t num_blocks, int32_t max_blocks_per_seq,
                                                   int32_t max_context_len, float scale,
                                                   void* stream) {
  clear_error();
  const char* fn = "paged_attention_decode_noalloc";
  int st = check_common(fn, batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_blocks_per_seq, max_context_len);
  if (st) return st;
  if (batch == 0) return GPKV_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return fail(GPKV_ERR_NULL, "%s: null pointer argument", fn);
  // The split-KV partial rows and the sequence prefix live in `scratch`. Nothing in
  // it has to start at zero: every call writes what its combine reads.
  const size_t need = gpkv_paged_attention_workspace_bytes(batch, num_q_heads, num_kv_heads,
                                                           head_dim, block_size, max_context_len);
  if (need > (size_t)GPKV_NOALLOC_SCRATCH_BYTES)
    return fail(GPKV_ERR_WORKSPACE,
                "%s: these sizes need %zu bytes of scratch, more than the library's fixed "
                "%zu-byte device array; use gpkv_paged_attention_decode with a workspace",
                fn, need, (size_t)GPKV_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_address(fn, &ws);
  if (st) return st;
  return attn_run(false, false, out, query, key_cache, value_cache, nullptr, nullptr,
                  block_tables, context_lens, nullptr, batch, num_q_heads, num_kv_heads, head_dim,
                  block_size, num_blocks, max_blocks_per_seq, max_context_len, 0, scale, ws,
                  (size_t)GPKV_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream);
}

extern "C" int gpkv_sparse_paged_attention_decode(
    float* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* topk_indices,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t topk_blocks, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return attn_run(true, false, out, query, key_cache, value_cache, nullptr, nullptr,
                  block_tables, context_lens, topk_indices, batch, num_q_heads, num_kv_heads,
                  head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                  topk_blocks, scale, workspace, workspace_bytes, (hipStream_t)stream);
}

extern "C" int gpkv_paged_attention_decode_fp8(
    float* out, const void* query, const void* key_cache, const void* value_cache,
    const float* k_scale, const float* v_scale, const int32_t* block_tables,
    const int32_t* context_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return attn_run(false, true, out, query, key_cache, value_cache, k_scale, v_scale,
                  block_tables, context_lens, nullptr, batch, num_q_heads, num_kv_heads, head_dim,
                  block_size, num_blocks, max_blocks_per_seq, max_context_len, 0, scale,
                  workspace, workspace_bytes, (hipStream_t)stream);
}

extern "C" int gpkv_sparse_paged_attention_decode_fp8(
    float* out, const void* query, const void* key_cache, const void* value_cache,
    const float* k_scale, const float* v_scale, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* topk_indices, int32_t batch, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t topk_blocks, float scale,
    void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return attn_run(true, true, out, query, key_cache, value_cache, k_scale, v_scale,
                  block_tables, context_lens, topk_indices, batch, num_q_heads, num_kv_heads,
                  head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                  topk_blocks, scale, workspace, workspace_bytes, (hipStream_t)stream);
}
