// Attention inner loop shared by the decode, sparse, multi-token and one-call Quest
// kernels, and the host helpers they share.
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
// Per-head inner loop (attend_head)
// ---------------------------------
// A wave handles one KV head g over a run of 16-token sub-tiles, two at a time
// (a 32-token tile). A sub-tile always lies inside one physical block
// (block_size is a multiple of 16), so its block id is wave-uniform and its rows
// are one contiguous region. The group's G query heads are padded to 16 and both
// contractions run on MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation:
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
// never pass through LDS. Rolling prefetch: the next tile's K is requested as
// soon as the current K has fed the q.k MFMAs, and its V right after the P.V
// MFMAs, so a wave keeps KV bytes in flight while it computes.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "gpkv_internal.h"

namespace gpkv {

constexpr int kWaves = 4;               // waves per workgroup
constexpr int kMaxTable = 2048;         // split path: block-table entries staged in LDS
constexpr int kMaxBalBatch = 4096;      // balanced path: largest batch (prefix in LDS)
constexpr int kMaxSubPerWG = 2048;      // balanced path: most sub-tiles per workgroup (dense)
constexpr int kBalTab = 4096;           // balanced path: table entries staged in LDS
constexpr int kDirTab = 2048;           // direct sparse path: longest Top-K list
constexpr int kCombineThreads = 256;   // combine kernels

struct AttnCommon {
  const unsigned short* q;   // [B, H_q, D] bf16
  const unsigned char* kc;   // [NB, bs, H_kv, D] bf16 or E4M3 codes
  const unsigned char* vc;
  const float* k_scale;      // [H_kv] (E4M3 caches only)
  const float* v_scale;
  long long block_bytes;     // bs * H_kv * D * element bytes
  int row_bytes;             // H_kv * D * element bytes
  int Hq, Hkv, G, bs;
  float qk_scale_log2;       // softmax scale * log2(e)
};

template <int D>
struct VecT;
template <>
struct VecT<128> {
  typedef u32x4 type;
  template <int AUX>
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return buf_load16<AUX>(r, off);
  }
};
template <>
struct VecT<64> {
  typedef u32x2 type;
  template <int AUX>
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return buf_load8<AUX>(r, off);
  }
};

// Channel of contraction slot j (< 8) of k-step s in lane group qd. bf16 caches:
// 32s + 8qd + j, so one 16-byte load per k-step. E4M3 caches: k-steps pair up
// (s = 2t + h) on 64t + 16qd + 8h + j, so one 16-byte load of codes serves two
// k-steps. The query operand follows the same order.
template <bool FP8>
__device__ __forceinline__ int kstep_channel(int s, int qd) {
  return FP8 ? 64 * (s >> 1) + 16 * qd + 8 * (s & 1) : 32 * s + 8 * qd;
}

// E4M3 code words -> bf16 operands: 16 codes (u32x4) give two k-step operands;
// one token's CPL codes give its V^T slice.
__device__ __forceinline__ void k_codes_to_bf16(u32x4 w, u32x4& s0, u32x4& s1) {
  const u32x2 a = e4m3x4_to_bf16(w[0]), b = e4m3x4_to_bf16(w[1]);
  const u32x2 c = e4m3x4_to_bf16(w[2]), d = e4m3x4_to_bf16(w[3]);
  s0 = u32x4{a[0], a[1], b[0], b[1]};
  s1 = u32x4{c[0], c[1], d[0], d[1]};
}
template <int D>
struct VCodes;
template <>
struct VCodes<128> {   // 8 codes per token
  typedef u32x2 type;
  template <int AUX>
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return buf_load8<AUX>(r, off);
  }
  static __device__ __forceinline__ u32x4 to_bf16(type w) {
    const u32x2 a = e4m3x4_to_bf16(w[0]), b = e4m3x4_to_bf16(w[1]);
    return u32x4{a[0], a[1], b[0], b[1]};
  }
};
template <>
struct VCodes<64> {    // 4 codes per token
  typedef unsigned type;
  template <int AUX>
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return buf_load4<AUX>(r, off);
  }
  static __device__ __forceinline__ u32x2 to_bf16(type w) { return e4m3x4_to_bf16(w); }
};

// RT tiles of up to 16 query rows that share every loaded K / V tile. For tile t,
// lane row r (= lane % 16): q[t] is the row's query (nullptr: a padding row of
// zeros), limit[t] its causal bound (CAUSAL only); rows r < n_rows[t] are written
// to o[t][r][D] (normalised) and lse[t][r] (base-2 log-sum-exp).
template <int RT>
struct RowTiles {
  const unsigned short* q[RT];
  int n_rows[RT];
  int limit[RT];
  float* o[RT];
  float* lse[RT];
};

// Attention of RT row tiles against KV head g over sub-tiles [0, n_sub) of one
// unit. Decode: one tile, the G query heads of the group. CAUSAL (multi-token
// queries): sub-tile u covers positions pos0 + 16u .., and a row sees only the
// positions below its bound; several row tiles per wave multiply the MFMA work
// done per K / V byte loaded.
template <int D, bool FP8, bool CAUSAL, int RT, class Desc>
__device__ __forceinline__ void attend_head(const AttnCommon& c, int g, int n_sub, const Desc& desc,
                                            int pos0, const RowTiles<RT>& rows) {
  constexpr int KSTEPS = D / 32;  // k-steps of the q.k contraction
  constexpr int KLOADS = FP8 ? D / 64 : KSTEPS;   // 16-byte K loads per sub-tile
  constexpr int CPL = D / 16;     // channels per lane in the V^T operand / O^T tiles
  constexpr int EB = FP8 ? 1 : 2; // bytes per cached element
  // Non-temporal loads: decode reads every K / V byte once, and so does a
  // multi-token unit on this per-head path (chunks long enough to re-read K / V
  // across many row tiles take the LDS-shared path, whose loads stay cached). On the
  // 8K-average caches, 58 single-token rows alone: 258 -> 192 us with them.
  constexpr int AUX = kLoadNT;
  typedef typename VecT<D>::type vvec;
  typedef typename VCodes<D>::type vcodes;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, qd = lane >> 4;
  // E4M3 caches: K's scale joins the softmax scale, V's scales the output.
  float qk_scale = c.qk_scale_log2, v_scale = 1.f;
  if constexpr (FP8) {
    qk_scale *= c.k_scale[g];
    v_scale = c.v_scale[g];
  }

  // Q^T operands: lane holds row r's channels of each k-step (zero for padding rows).
  u32x4 qf[RT][KSTEPS];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    if (rows.q[t] != nullptr) {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        qf[t][s] = *(const u32x4*)(rows.q[t] + kstep_channel<FP8>(s, qd));
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[t][s] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x4 oacc[RT][CPL];
  float m_run[RT], l_run[RT];  // running max of row r (base 2, same in its 4 lanes) and
                               // this lane's share of the normaliser
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) oacc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
  }

  const unsigned off_k = (unsigned)(r * c.row_bytes + g * D * EB + qd * 16);
  const unsigned off_v = (unsigned)(4 * qd * c.row_bytes + g * D * EB + r * CPL * EB);
  const int n_tiles = (n_sub + 1) >> 1;

  auto describe = [&](int k, int* pb, int* row0, int* nv) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int u = 2 * k + sub;
      if (u < n_sub) {
        desc(u, pb[sub], row0[sub], nv[sub]);
      } else {
        pb[sub] = 0;
        row0[sub] = 0;
        nv[sub] = 0;
      }
    }
  };
  // The next tile with at least one valid row, or n_tiles with an empty
  // descriptor (nv = 0, so loads issued for it read nothing).
  auto next_tile = [&](int k, int* pb, int* row0, int* nv) {
    for (; k < n_tiles; ++k) {
      describe(k, pb, row0, nv);
      if ((nv[0] | nv[1]) != 0) return k;
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      pb[sub] = 0;
      row0[sub] = 0;
      nv[sub] = 0;
    }
    return n_tiles;
  };

  // In flight: bf16 operands (kf, vf), or E4M3 codes (kq, vq) converted to bf16
  // operands right before their MFMAs.
  u32x4 kf[2][KSTEPS];
  vvec vf[2][4];
  u32x4 kq[2][KLOADS];
  vcodes vq[2][4];
  auto issue_k = [&](const int* pb, const int* row0, const int* nv) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const size_t base = (size_t)pb[sub] * (size_t)c.block_bytes + (size_t)row0[sub] * c.row_bytes;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(c.kc + base, (unsigned)(nv[sub] * c.row_bytes));
#pragma unroll
      for (int s = 0; s < KLOADS; ++s) {
        if constexpr (FP8)
          kq[sub][s] = buf_load16<AUX>(rk, off_k + 64 * s);
        else
          kf[sub][s] = buf_load16<AUX>(rk, off_k + 64 * s);
      }
    }
  };
  auto issue_v = [&](const int* pb, const int* row0, const int* nv) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const size_t base = (size_t)pb[sub] * (size_t)c.block_bytes + (size_t)row0[sub] * c.row_bytes;
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(c.vc + base, (unsigned)(nv[sub] * c.row_bytes));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (FP8)
          vq[sub][i] = VCodes<D>::template load<AUX>(rv, off_v + i * c.row_bytes);
        else
          vf[sub][i] = VecT<D>::template load<AUX>(rv, off_v + i * c.row_bytes);
      }
    }
  };

  // Loads are issued unconditionally (an empty descriptor past the last tile
  // reads nothing): with a load issued on only some paths, the compiler's
  // wait-count merge would make the P.V step wait for the prefetched K as well.
  // The next tile's descriptor is found one tile ahead, so its table reads are
  // off the path between the q.k MFMAs and the K prefetch.
  int pb[2], row0[2], nv[2], pbn[2], row0n[2], nvn[2];
  int k = next_tile(0, pb, row0, nv);
  int kn = next_tile(k + 1, pbn, row0n, nvn);
  // K before V on every path into the loop (the scheduler may not swap them),
  // so waiting for K at the top of an iteration leaves V in flight.
  issue_k(pb, row0, nv);
  __builtin_amdgcn_sched_barrier(0);
  issue_v(pb, row0, nv);
  __builtin_amdgcn_sched_barrier(0);
  while (k < n_tiles) {
    if constexpr (FP8) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int t = 0; t < KLOADS; ++t) k_codes_to_bf16(kq[sub][t], kf[sub][2 * t], kf[sub][2 * t + 1]);
    }
    // S^T for both sub-tiles.
    f32x4 sacc[RT][2];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        sacc[t][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
          sacc[t][sub] = mfma16x16x32(kf[sub][s], qf[t][s], sacc[t][sub]);
      }
    issue_k(pbn, row0n, nvn);

    // Online softmax over this tile for row r of each row tile (base 2), and the
    // P^T operands as bf16 hi + lo parts.
    u32x4 phi[RT], plo[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      float sv[8];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = sacc[t][sub][i] * qk_scale;
          bool ok = 4 * qd + i < nv[sub];
          if constexpr (CAUSAL)
            ok = ok && pos0 + 16 * (2 * k + sub) + 4 * qd + i < rows.limit[t];
          sv[sub * 4 + i] = ok ? x : -INFINITY;
        }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
      mx = max_across_rows(mx);
      const float m_new = fmaxf(m_run[t], mx);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_ref);
      float pv[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_ref);
        psum += pv[i];
      }
      l_run[t] = l_run[t] * alpha + psum;
      m_run[t] = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) oacc[t][j] *= alpha;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const unsigned a = __float_as_uint(pv[2 * d]), cc = __float_as_uint(pv[2 * d + 1]);
        phi[t][d] = pack_hi16(a, cc);
        const float ra = pv[2 * d] - __uint_as_float(a & 0xffff0000u);
        const float rc = pv[2 * d + 1] - __uint_as_float(cc & 0xffff0000u);
        plo[t][d] = pack_hi16(__float_as_uint(ra), __float_as_uint(rc));
      }
    }

    if constexpr (FP8) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[sub][i] = VCodes<D>::to_bf16(vq[sub][i]);
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
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        oacc[t][j] = mfma16x16x32(va, phi[t], oacc[t][j]);
        oacc[t][j] = mfma16x16x32(va, plo[t], oacc[t][j]);
      }
    }
    issue_v(pbn, row0n, nvn);
    k = kn;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      pb[sub] = pbn[sub];
      row0[sub] = row0n[sub];
      nv[sub] = nvn[sub];
    }
    kn = next_tile(k + 1, pbn, row0n, nvn);
  }

  // The unit's result per row tile: normalised output and base-2 log-sum-exp.
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const float l_tot = sum_across_rows(l_run[t]);
    if (r < rows.n_rows[t]) {
      const float inv = l_tot > 0.f ? v_scale / l_tot : 0.f;
      float* dst = rows.o[t] + (size_t)r * D + CPL * 4 * qd;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j0 = 0; j0 < CPL; j0 += 4) {
          f32x4 v;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v[jj] = oacc[t][j0 + jj][i] * inv;
          *(f32x4*)(dst + CPL * i + j0) = v;
        }
      }
      if (qd == 0) rows.lse[t][r] = l_tot > 0.f ? m_run[t] + log2f(l_tot) : -INFINITY;
    }
  }
}

// A merge of partial rows in progress: acc and W are relative to mr (-inf: nothing
// merged yet).
struct MergeState {
  f32x4 acc;
  float W, mr;
};

// One more row (base-2 lse l, normalised values v) into a merge.
__device__ __forceinline__ void merge_one(MergeState& st, float l, const f32x4& v) {
  const float m = fmaxf(st.mr, l);
  if (m == -INFINITY) return;
  const float s = __builtin_amdgcn_exp2f(st.mr - m);   // 0 when mr = -inf
  const float w = __builtin_amdgcn_exp2f(l - m);
  st.W = st.W * s + w;
  st.acc = st.acc * s + w * v;
  st.mr = m;
}

__device__ __forceinline__ f32x4 merge_finish(const MergeState& st) {
  const float inv = st.W > 0.f ? 1.f / st.W : 0.f;
  return st.acc * inv;
}

// Merge of n partial rows (one float4 column of each): row k has base-2 lse
// lse0[k * ls] and normalised output o0[k * os]; live(k) false skips a row.
// merge_rows returns sum_k 2^(lse_k - M) O_k / sum_k 2^(lse_k - M) (zeros when no
// row holds a token). NU rows (lse and output) are requested together, and the sum
// is kept relative to the largest lse seen so far, so up to NU rows cost one round
// of loads.
template <int NU, class Live>
__device__ __forceinline__ MergeState merge_rows_state(int n, const float* lse0, size_t ls,
                                                       const float* o0, size_t os,
                                                       const Live& live) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f, mr = -INFINITY;   // acc and W are relative to mr (-inf: nothing yet)
  for (int k0 = 0; k0 < n; k0 += NU) {
    float l[NU];
    f32x4 v[NU];
#pragma unroll
    for (int x = 0; x < NU; ++x) {
      const int k = k0 + x;
      const bool ok = k < n && live(k);
      l[x] = ok ? lse0[(size_t)k * ls] : -INFINITY;
      v[x] = ok ? *(const f32x4*)(o0 + (size_t)k * os) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m = mr;
#pragma unroll
    for (int x = 0; x < NU; ++x) m = fmaxf(m, l[x]);
    if (m == -INFINITY) continue;
    const float s = __builtin_amdgcn_exp2f(mr - m);   // 0 when mr = -inf
    W *= s;
    acc *= s;
    mr = m;
#pragma unroll
    for (int x = 0; x < NU; ++x) {
      const float w = __builtin_amdgcn_exp2f(l[x] - m);   // 0 for skipped rows
      W += w;
      acc += w * v[x];
    }
  }
  return MergeState{acc, W, mr};
}

template <int NU, class Live>
__device__ __forceinline__ f32x4 merge_rows(int n, const float* lse0, size_t ls, const float* o0,
                                            size_t os, const Live& live) {
  return merge_finish(merge_rows_state<NU>(n, lse0, ls, o0, os, live));
}

__device__ __forceinline__ int clamp_ctx(int v, int max_ctx) {
  return v < 0 ? 0 : (v > max_ctx ? max_ctx : v);
}

// Decode append (the step's cache write merged into the decode call): sequence b's
// newest token, at position ctx - 1, comes from the call's key / value inputs when
// its slot lies in the pool and the context holds it. The split phase then stops
// one position short and the combine merges the token as one more unit.
// The slot is requested together with the context length (not after it), so that
// neither load waits for the other.
__device__ __forceinline__ bool append_token(const long long* slots, long long num_slots, int b,
                                             const int* ctx, int max_ctx) {
  if (slots == nullptr) return false;
  const long long s = slots[b];
  const int c = clamp_ctx(ctx[b], max_ctx);
  return c >= 1 && s >= 0 && s < num_slots;
}
// Decode append: KV head g's part of sequence b's new token written into the cache at
// slot s (0 <= s < NB * bs) and, when kmin is non-null, folded into its block's Quest
// key min / max (row 0 of a block starts it afresh), as the write path does. The
// calling threads split the D / 8 16-byte vectors of the row.
template <int D>
__device__ __forceinline__ void store_new_token(const unsigned short* knew,
                                                const unsigned short* vnew, unsigned short* kc,
                                                unsigned short* vc, unsigned short* kmin,
                                                unsigned short* kmax, long long s, int bs, int Hkv,
                                                int b, int g, int t, int nt) {
  const long long blk = s / bs, off = s - blk * bs;
  const size_t row = (size_t)Hkv * D;   // bf16 per cache row
  for (int c = t; c < D / 8; c += nt) {
    const size_t src = ((size_t)b * Hkv + g) * D + 8 * c;
    const size_t dst = (size_t)s * row + (size_t)g * D + 8 * c;
    const u32x4 k = *(const u32x4*)(knew + src);
    *(u32x4*)(kc + dst) = k;
    *(u32x4*)(vc + dst) = *(const u32x4*)(vnew + src);
    if (kmin != nullptr) {
      const size_t meta = (size_t)blk * row + (size_t)g * D + 8 * c;
      u32x4 mn = k, mx = k;
      if (off > 0) fold_min_max(k, *(const u32x4*)(kmin + meta), *(const u32x4*)(kmax + meta), mn, mx);
      *(u32x4*)(kmin + meta) = mn;
      *(u32x4*)(kmax + meta) = mx;
    }
  }
}

// store_new_token for E4M3 caches: KV head g's part of the token quantised as the
// FP8 write path quantises it (code = e4m3(x * (1 / scale[g]))), and its key codes
// folded into E4M3 metadata. The calling threads split the D / 16 16-byte code
// vectors of the row.
template <int D>
__device__ __forceinline__ void store_new_token_fp8(const unsigned short* knew,
                                                    const unsigned short* vnew, unsigned char* kc,
                                                    unsigned char* vc, unsigned char* kmin,
                                                    unsigned char* kmax, const float* k_scale,
                                                    const float* v_scale, long long s, int bs,
                                                    int Hkv, int b, int g, int t, int nt) {
  const long long blk = s / bs, off = s - blk * bs;
  const size_t row = (size_t)Hkv * D;   // bytes per cache row
  const float kinv = 1.0f / k_scale[g], vinv = 1.0f / v_scale[g];
  for (int c = t; c < D / 16; c += nt) {
    const u32x4* ks = (const u32x4*)(knew + ((size_t)b * Hkv + g) * D + 16 * c);
    const u32x4* vs = (const u32x4*)(vnew + ((size_t)b * Hkv + g) * D + 16 * c);
    const size_t dst = (size_t)s * row + (size_t)g * D + 16 * c;
    const u32x4 k = quantize16(ks[0], ks[1], kinv);
    *(u32x4*)(kc + dst) = k;
    *(u32x4*)(vc + dst) = quantize16(vs[0], vs[1], vinv);
    if (kmin != nullptr) {
      const size_t meta = (size_t)blk * row + (size_t)g * D + 16 * c;
      u32x4 mn = k, mx = k;
      if (off > 0) fold_min_max_e4m3(k, *(const u32x4*)(kmin + meta), *(const u32x4*)(kmax + meta), mn, mx);
      *(u32x4*)(kmin + meta) = mn;
      *(u32x4*)(kmax + meta) = mx;
    }
  }
}

// Positions of sequence b the split phase reads: its clamped context, less the
// appended token.
__device__ __forceinline__ int split_ctx(const int* ctx, const long long* slots,
                                         long long num_slots, int b, int max_ctx) {
  const long long s = slots != nullptr ? slots[b] : -1;
  const int c = clamp_ctx(ctx[b], max_ctx);
  return c - ((c >= 1 && s >= 0 && s < num_slots) ? 1 : 0);
}


// Exclusive prefix sum over the workgroup's NW * 64 threads; *total gets the sum.
template <int NW = kWaves>
__device__ __forceinline__ int wg_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = (int)wave_inclusive_scan((unsigned)v);
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = s_wave[w];
    off += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// Host side, defined in paged_attention.hip.
size_t align256(size_t x);
// Argument checks every attention entry point shares (status, message set).
int check_common(const char* fn, int B, int Hq, int Hkv, int D, int bs, long long NB,
                 int max_blocks, int max_ctx);

}  // namespace gpkv
