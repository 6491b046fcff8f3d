// GQA paged decode attention, dense and Quest-sparse: split-KV partials + combine.
//
// What is computed (["Ascend Kernel-to-Serving Pipeline", sections "GQA Paged
// Attention" and "Quest Sparse Attention"]): for each sequence b and query head h,
// softmax attention of q[b,h] over the tokens of b (all tokens < context_lens[b],
// or only those in the selected logical blocks), reading K/V of KV head
// h / G through block_tables, the ragged last block masked. The running max /
// normaliser / rescaled accumulator (online softmax) and the split + weighted
// combine ([TL18] = TileLang tutorial ch. 18, section 4.1) are how the kernel
// reaches that result; they are not a different definition.
//
// Work decomposition (MI355X-first)
// ---------------------------------
// A workgroup owns one (sequence b, split) unit: a range of `split_tokens` tokens
// (dense) or of selected-block tokens (sparse), for every KV head. Its waves each
// take one KV head (wave w: heads w, w + W, ...), so the waves stream the same
// token rows at the same time: on MI355X whole cache rows (all KV heads of a
// token) then come from HBM together, which sustains more bandwidth than
// scattering the heads of a row over different workgroups. A wave walks the
// split's 32-token tiles; each tile is two 16-token sub-tiles, and a 16-token
// sub-tile always lies inside one physical block (block_size is a multiple of
// 16), so its block id is wave-uniform and its rows are one contiguous region.
//
// The group's G query heads are padded to 16 and both contractions run on MFMA
// (v_mfma_f32_16x16x32_bf16) with fp32 accumulation:
//   S^T[t, h] = sum_c K[t, c] Q[h, c]          A = K rows, B = Q^T
//   O^T[c, h] += sum_t V^T[c, t] P^T[t, h]      A = V^T,   B = P^T
// Lane (r = lane % 16, qd = lane / 16) supplies A/B row or column r and the
// eight contraction slots 8*qd..8*qd+7. The contraction order is free, so:
//   - K: lane loads token r's channels 32s + 8qd .. +8 (16 B) for k-step s;
//   - S^T lands as head r x tokens {4qd+i} of each sub-tile, which is exactly the
//     slot set the P^T operand needs (slots 0-3: sub-tile 0, 4-7: sub-tile 1);
//   - V^T row r of tile j is channel CPL*r + j (CPL = D/16), so the lane's eight
//     V values per tile come from the rows of its own eight tokens, channels
//     CPL*r .. CPL*r+CPL: one 16-byte (D=128) load per token, repacked with
//     v_perm -- no LDS transpose.
// P is fed as a bf16 hi + lo pair (two MFMAs), so the only rounding of the
// weights is the ~2^-16 relative truncation of the low part.
// Masking uses raw buffer loads whose descriptor ends after the sub-tile's valid
// rows: rows past the context read as zeros (never NaN), and their scores are
// set to -inf. KV loads are non-temporal (each byte is read once per step) and
// never pass through LDS; LDS holds only the split's block-table entries.
#include <math.h>

#include "gpkv_internal.h"

namespace gpkv {

constexpr int kMaxWaves = 8;            // waves per workgroup (KV heads processed at once)
constexpr int kMaxSplitTokens = 2048;
constexpr int kMaxTable = 2048;         // block-table entries staged in LDS per workgroup

struct SplitParams {
  float* part_o;             // [B, H_kv, S, G, D] fp32, each split's normalised output
  float* part_lse;           // [B, H_kv, S, G] fp32, base-2 log-sum-exp of the split
  const unsigned short* q;   // [B, H_q, D] bf16
  const unsigned char* kc;   // [NB, bs, H_kv, D] bf16
  const unsigned char* vc;
  const int* block_tables;   // [B, max_blocks]
  const int* ctx;            // [B]
  const int* topk;           // [B, H_kv, K] (sparse only)
  long long block_bytes;     // bs * H_kv * D * 2
  int row_bytes;             // H_kv * D * 2
  long long NB;              // pool size; block ids outside [0, NB) select nothing
  int Hq, Hkv, G, bs, max_blocks, max_ctx, num_splits, split_tokens, topk_blocks;
  float qk_scale_log2;       // softmax scale * log2(e)
};

template <int D>
struct VecT;
template <>
struct VecT<128> {
  typedef u32x4 type;
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return buf_load16(r, off);
  }
};
template <>
struct VecT<64> {
  typedef u32x2 type;
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return buf_load8(r, off);
  }
};

template <int D, bool SPARSE>
__global__ __launch_bounds__(kMaxWaves * 64) void attn_split_kernel(const SplitParams p) {
  constexpr int KSTEPS = D / 32;  // k-steps of the q.k contraction
  constexpr int CPL = D / 16;     // channels per lane in the V^T operand / O^T tiles
  constexpr int VBYTES = CPL * 2;
  typedef typename VecT<D>::type vvec;

  // Block-table entries of the split: entry e covers virtual tokens
  // [t0 + e*bs, t0 + (e+1)*bs). s_tok0 = logical position of the block's row 0,
  // or a huge value when the entry selects nothing. Dense: one table shared by all
  // KV heads; sparse: one table per KV head (the selection is per head).
  __shared__ int s_pb[kMaxTable];
  __shared__ int s_tok0[kMaxTable];

  const int split = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int W = blockDim.x >> 6;
  const int wave = uniform(tid >> 6);  // tell the compiler the tile loop is wave-uniform
  const int r = lane & 15, qd = lane >> 4;
  const int G = p.G, bs = p.bs, Hkv = p.Hkv;
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);  // memory safety only
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
    s_pb[i] = ok ? pb : 0;
    s_tok0[i] = ok ? lb * bs : 0x3fffffff;
  }
  __syncthreads();

  const int n_tiles = T / 32;
  for (int g = wave; g < Hkv; g += W) {
    const int* tab_pb = s_pb + (SPARSE ? g * n_ent : 0);
    const int* tab_t0 = s_tok0 + (SPARSE ? g * n_ent : 0);

    // Q^T operand: lane holds head r's channels 32s + 8qd .. +8 (zero rows past G).
    u32x4 qf[KSTEPS];
    if (r < G) {
      const unsigned short* qrow = p.q + ((size_t)b * p.Hq + (size_t)g * G + r) * D;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[s] = *(const u32x4*)(qrow + 32 * s + 8 * qd);
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[s] = u32x4{0u, 0u, 0u, 0u};
    }

    f32x4 oacc[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max of head r (base 2), same in its 4 lanes
    float l_run = 0.f;        // this lane's share of the normaliser

    const unsigned off_k = (unsigned)(r * p.row_bytes + g * D * 2 + qd * 16);
    const unsigned off_v = (unsigned)(4 * qd * p.row_bytes + g * D * 2 + r * VBYTES);

    // Tile k covers sub-tiles 2k and 2k+1. For each sub-tile: physical block,
    // first row inside it, number of valid rows (all wave-uniform).
    auto describe = [&](int k, int* pb, int* row0, int* nv) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int u16 = 16 * (2 * k + sub);
        const int e = u16 / bs;
        row0[sub] = u16 & (bs - 1);
        int n = ctx - (tab_t0[e] + row0[sub]);
        n = n < 0 ? 0 : (n > 16 ? 16 : n);
        nv[sub] = uniform(n);
        pb[sub] = uniform(tab_pb[e]);
      }
    };
    // The next tile with at least one valid row, or n_tiles. Dense tiles are
    // contiguous from the split start, so the first empty one ends the split;
    // a sparse list may have unselected entries anywhere.
    auto next_tile = [&](int k, int* pb, int* row0, int* nv) {
      for (; k < n_tiles; ++k) {
        describe(k, pb, row0, nv);
        if ((nv[0] | nv[1]) != 0) return k;
        if (!SPARSE) return n_tiles;
      }
      return n_tiles;
    };

    u32x4 kf[2][KSTEPS];
    vvec vf[2][4];
    auto issue_k = [&](const int* pb, const int* row0, const int* nv) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const size_t base = (size_t)pb[sub] * (size_t)p.block_bytes + (size_t)row0[sub] * p.row_bytes;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.kc + base, (unsigned)(nv[sub] * p.row_bytes));
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) kf[sub][s] = buf_load16(rk, off_k + 64 * s);
      }
    };
    auto issue_v = [&](const int* pb, const int* row0, const int* nv) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const size_t base = (size_t)pb[sub] * (size_t)p.block_bytes + (size_t)row0[sub] * p.row_bytes;
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.vc + base, (unsigned)(nv[sub] * p.row_bytes));
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[sub][i] = VecT<D>::load(rv, off_v + i * p.row_bytes);
      }
    };

    // Rolling prefetch: the next tile's K is requested as soon as the current K
    // has fed the q.k MFMAs, and its V right after the P.V MFMAs, so the wave
    // keeps KV bytes in flight while it computes.
    int pb[2], row0[2], nv[2];
    int k = next_tile(0, pb, row0, nv);
    if (k < n_tiles) {
      issue_k(pb, row0, nv);
      issue_v(pb, row0, nv);
    }
    while (k < n_tiles) {
      // S^T for both sub-tiles.
      f32x4 sacc[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        sacc[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) sacc[sub] = mfma16x16x32(kf[sub][s], qf[s], sacc[sub]);
      }
      int pbn[2], row0n[2], nvn[2];
      const int kn = next_tile(k + 1, pbn, row0n, nvn);
      if (kn < n_tiles) issue_k(pbn, row0n, nvn);

      // Online softmax over this tile for head r (base 2).
      float sv[8];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = sacc[sub][i] * p.qk_scale_log2;
          sv[sub * 4 + i] = (4 * qd + i < nv[sub]) ? x : -INFINITY;
        }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
      float pv[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_ref);
        psum += pv[i];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) oacc[j] *= alpha;
      }

      // P^T operand as bf16 hi + lo parts.
      u32x4 phi, plo;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const unsigned a = __float_as_uint(pv[2 * d]), c = __float_as_uint(pv[2 * d + 1]);
        phi[d] = pack_hi16(a, c);
        const float ra = pv[2 * d] - __uint_as_float(a & 0xffff0000u);
        const float rc = pv[2 * d + 1] - __uint_as_float(c & 0xffff0000u);
        plo[d] = pack_hi16(__float_as_uint(ra), __float_as_uint(rc));
      }

      // O^T += V^T P^T, one 16-channel tile j at a time.
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        u32x4 va;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int sub = d >> 1, i0 = (d & 1) * 2;
          const unsigned w0 = vf[sub][i0][j >> 1], w1 = vf[sub][i0 + 1][j >> 1];
          va[d] = (j & 1) ? pack_hi16(w0, w1) : pack_lo16(w0, w1);
        }
        oacc[j] = mfma16x16x32(va, phi, oacc[j]);
        oacc[j] = mfma16x16x32(va, plo, oacc[j]);
      }
      if (kn < n_tiles) issue_v(pbn, row0n, nvn);
      k = kn;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        pb[sub] = pbn[sub];
        row0[sub] = row0n[sub];
        nv[sub] = nvn[sub];
      }
    }

    // This head's split result: normalised output and base-2 log-sum-exp.
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const size_t unit = ((size_t)b * Hkv + g) * p.num_splits + split;
    if (r < G) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      float* dst = p.part_o + (unit * G + r) * D + CPL * 4 * qd;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j0 = 0; j0 < CPL; j0 += 4) {
          f32x4 v;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v[jj] = oacc[j0 + jj][i] * inv;
          *(f32x4*)(dst + CPL * i + j0) = v;
        }
      }
      if (qd == 0) p.part_lse[unit * G + r] = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
    }
  }
}

struct CombineParams {
  float* out;               // [B, H_q, D]
  const float* part_o;
  const float* part_lse;
  const int* ctx;
  int Hq, Hkv, G, max_ctx, num_splits, split_tokens, sparse;
};

// out = sum_s w_s O_s / sum_s w_s with w_s = 2^(lse_s - max lse): each split's
// normaliser taken relative to one common maximum ([TL18] 4.1). One wave per
// (sequence, query head).
template <int D>
__global__ __launch_bounds__(64) void attn_combine_kernel(const CombineParams p) {
  constexpr int CP = D / 64;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int G = p.G;
  const int g = h / G, hl = h - g * G;
  int ctx = p.ctx[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int ns = p.sparse ? p.num_splits : (ctx + p.split_tokens - 1) / p.split_tokens;
  const size_t unit0 = ((size_t)b * p.Hkv + g) * p.num_splits;
  const float* lse = p.part_lse + unit0 * G + hl;
  const float* po = p.part_o + unit0 * (size_t)G * D + (size_t)hl * D + lane * CP;

  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, lse[(size_t)s * G]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float Mr = (M == -INFINITY) ? 0.f : M;

  float acc[CP];
#pragma unroll
  for (int c = 0; c < CP; ++c) acc[c] = 0.f;
  float W = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = __builtin_amdgcn_exp2f(lse[(size_t)s * G] - Mr);
    W += w;
    const float* src = po + (size_t)s * G * D;
#pragma unroll
    for (int c = 0; c < CP; ++c) acc[c] += w * src[c];
  }
  float* o = p.out + ((size_t)b * p.Hq + h) * D + lane * CP;
#pragma unroll
  for (int c = 0; c < CP; ++c) o[c] = (W > 0.f) ? acc[c] / W : 0.f;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  int split_tokens, num_splits;
  size_t o_bytes, lse_bytes;
};

static int waves_per_wg(int Hkv) { return Hkv < kMaxWaves ? Hkv : kMaxWaves; }

static Plan make_plan(bool sparse, int B, int Hq, int Hkv, int D, int bs, int span) {
  Plan pl;
  const int G = Hq / Hkv;
  pl.split_tokens = split_tokens_for(B, Hkv, span);
  // The split's block-table entries (per KV head when sparse) must fit in LDS.
  const int per_token_entries = sparse ? Hkv : 1;
  while (pl.split_tokens > 128 && (pl.split_tokens / bs) * per_token_entries > kMaxTable)
    pl.split_tokens >>= 1;
  pl.num_splits = (span + pl.split_tokens - 1) / pl.split_tokens;
  if (pl.num_splits < 1) pl.num_splits = 1;
  const size_t units = (size_t)B * Hkv * pl.num_splits;
  pl.o_bytes = align256(units * G * D * sizeof(float));
  pl.lse_bytes = align256(units * G * sizeof(float));
  return pl;
}

static int check_common(const char* fn, int B, int Hq, int Hkv, int D, int bs, long long NB,
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

static int attn_run(bool sparse, float* out, const void* query, const void* kc, const void* vc,
                    const int* bt, const int* ctx, const int* topk, int B, int Hq, int Hkv, int D,
                    int bs, long long NB, int max_blocks, int max_ctx, int K, float scale,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = sparse ? "sparse_paged_attention_decode" : "paged_attention_decode";
  int st = check_common(fn, B, Hq, Hkv, D, bs, NB, max_blocks, max_ctx);
  if (st) return st;
  if (sparse && K < 1) return fail(GPKV_ERR_SHAPE, "%s: topk_blocks=%d < 1", fn, K);
  if (B == 0) return GPKV_OK;
  if (!out || !query || !kc || !vc || !bt || !ctx || (sparse && !topk))
    return fail(GPKV_ERR_NULL, "%s: null pointer argument", fn);
  const long long span_ll = sparse ? (long long)K * bs : (long long)max_ctx;
  if (span_ll > (1LL << 30)) return fail(GPKV_ERR_SHAPE, "%s: token span too large", fn);
  if (sparse && (128 / bs) * Hkv > kMaxTable)
    return fail(GPKV_ERR_UNSUPPORTED, "%s: num_kv_heads=%d too large for block_size %d", fn, Hkv, bs);
  const Plan pl = make_plan(sparse, B, Hq, Hkv, D, bs, (int)span_ll);
  const size_t need = pl.o_bytes + pl.lse_bytes;
  if (!ws || ws_bytes < need)
    return fail(GPKV_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn,
                ws ? ws_bytes : (size_t)0, need);

  const int G = Hq / Hkv;
  SplitParams sp;
  sp.part_o = (float*)ws;
  sp.part_lse = (float*)((char*)ws + pl.o_bytes);
  sp.q = (const unsigned short*)query;
  sp.kc = (const unsigned char*)kc;
  sp.vc = (const unsigned char*)vc;
  sp.block_tables = bt;
  sp.ctx = ctx;
  sp.topk = topk;
  sp.row_bytes = Hkv * D * 2;
  sp.block_bytes = (long long)bs * sp.row_bytes;
  sp.Hq = Hq;
  sp.Hkv = Hkv;
  sp.G = G;
  sp.bs = bs;
  sp.max_blocks = max_blocks;
  sp.max_ctx = max_ctx;
  sp.NB = NB;
  sp.num_splits = pl.num_splits;
  sp.split_tokens = pl.split_tokens;
  sp.topk_blocks = sparse ? K : 0;
  sp.qk_scale_log2 = scale * 1.4426950408889634f;

  const dim3 grid(pl.num_splits, B), block(64 * waves_per_wg(Hkv));
  if (D == 128) {
    if (sparse)
      attn_split_kernel<128, true><<<grid, block, 0, stream>>>(sp);
    else
      attn_split_kernel<128, false><<<grid, block, 0, stream>>>(sp);
  } else {
    if (sparse)
      attn_split_kernel<64, true><<<grid, block, 0, stream>>>(sp);
    else
      attn_split_kernel<64, false><<<grid, block, 0, stream>>>(sp);
  }
  st = check_launch(fn);
  if (st) return st;

  CombineParams cp;
  cp.out = out;
  cp.part_o = sp.part_o;
  cp.part_lse = sp.part_lse;
  cp.ctx = ctx;
  cp.Hq = Hq;
  cp.Hkv = Hkv;
  cp.G = G;
  cp.max_ctx = max_ctx;
  cp.num_splits = pl.num_splits;
  cp.split_tokens = pl.split_tokens;
  cp.sparse = sparse ? 1 : 0;
  const dim3 cgrid(Hq, B), cblock(64);
  if (D == 128)
    attn_combine_kernel<128><<<cgrid, cblock, 0, stream>>>(cp);
  else
    attn_combine_kernel<64><<<cgrid, cblock, 0, stream>>>(cp);
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
  return pl.o_bytes + pl.lse_bytes;
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
  return pl.o_bytes + pl.lse_bytes;
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
  return attn_run(false, out, query, key_cache, value_cache, block_tables, context_lens, nullptr,
                  batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                  max_blocks_per_seq, max_context_len, 0, scale, workspace, workspace_bytes,
                  (hipStream_t)stream);
}

extern "C" int gpkv_sparse_paged_attention_decode(
    float* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* topk_indices,
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t topk_blocks, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return attn_run(true, out, query, key_cache, value_cache, block_tables, context_lens,
                  topk_indices, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                  num_blocks, max_blocks_per_seq, max_context_len, topk_blocks, scale, workspace,
                  workspace_bytes, (hipStream_t)stream);
}
