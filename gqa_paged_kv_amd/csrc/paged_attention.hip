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
//
// Work decomposition (MI355X-first)
// ---------------------------------
// Workgroups hold 4 waves; the waves of a workgroup take different KV heads of
// the same tokens, so whole cache rows (every KV head of a token) stream from
// HBM together.
//  - Dense (balanced): the grid is one workgroup per compute unit. Each
//    workgroup computes the prefix sums of the sequences' 16-token sub-tile
//    counts and takes an equal share of the flattened (sequence, sub-tile)
//    space, so ragged batches cost no tail: every workgroup moves the same
//    number of KV bytes. A workgroup writes one partial per sequence it
//    touches into slot (workgroup + sequence), which is unique because shares are
//    ordered; the combine recomputes which workgroups covered a sequence.
//  - Sparse, and dense batches too large for the balanced table: a workgroup per
//    (sequence, split of `split_tokens` virtual tokens), the split's block-table
//    entries (per KV head when sparse) staged in LDS.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "gpkv_internal.h"
#include "quest_select.h"

namespace gpkv {

constexpr int kWaves = 4;               // waves per workgroup
constexpr int kMaxTable = 2048;         // split path: block-table entries staged in LDS
constexpr int kMaxBalBatch = 4096;      // balanced path: largest batch (prefix in LDS)
constexpr int kMaxSubPerWG = 2048;      // balanced path: most sub-tiles per workgroup (dense)
constexpr int kBalTab = 4096;           // balanced path: table entries staged in LDS
constexpr int kDirTab = 2048;           // direct sparse path: longest Top-K list

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

// Attention of the G query heads of KV head g over sub-tiles [0, n_sub) of one
// unit; `desc(u, pb, row0, nv)` names sub-tile u's physical block, first row and
// valid rows (nv = 0: nothing selected). Writes the unit's normalised output
// o_dst[h][D] and base-2 log-sum-exp lse_dst[h] for h < G.
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
  // Decode reads every K / V byte once: non-temporal loads. Multi-token queries
  // re-read a split's K / V from every row tile of the chunk: cached loads.
  constexpr int AUX = CAUSAL ? 0 : kLoadNT;
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
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
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
    float l_tot = l_run[t] + __shfl_xor(l_run[t], 16);
    l_tot += __shfl_xor(l_tot, 32);
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

// Causal rows of one KV head shared by the whole workgroup: each wave carries two
// row tiles, and every 32-token K / V tile is loaded once per workgroup into LDS
// (double-buffered, loads for the next tile in flight while this one is used)
// instead of once per wave. Same arithmetic as attend_head; every wave of the
// workgroup must call it with the same n_sub, desc and pos0 (it has barriers).
constexpr int kShareRowBytes(int D) { return 2 * D + 16; }   // padded LDS row
constexpr int kShareLdsBytes(int D) { return 2 * 2 * 32 * kShareRowBytes(D); }

template <int D, class Desc>
__device__ __forceinline__ void attend_shared(const AttnCommon& c, int g, int n_sub,
                                              const Desc& desc, int pos0, const RowTiles<2>& rows,
                                              unsigned char* s_kv) {
  constexpr int RT = 2;
  constexpr int KSTEPS = D / 32;
  constexpr int CPL = D / 16;
  constexpr int ROWB = kShareRowBytes(D);
  constexpr int TILEB = 32 * ROWB;           // one 32-token K or V tile in LDS
  constexpr int PIECES = 2 * D / 16;         // 16-byte pieces per token row
  constexpr int PER_T = 32 * PIECES / (kWaves * 64);   // pieces per thread per tile
  static_assert(PER_T >= 1 && 32 * PIECES == PER_T * kWaves * 64, "tile split");
  typedef typename VecT<D>::type vvec;
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = lane & 15, qd = lane >> 4;
  const bool active = rows.n_rows[0] > 0;   // the wave's second tile is empty if its first is

  u32x4 qf[RT][KSTEPS];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[t][s] = rows.q[t] != nullptr ? *(const u32x4*)(rows.q[t] + 32 * s + 8 * qd)
                                      : u32x4{0u, 0u, 0u, 0u};
  }
  f32x4 oacc[RT][CPL];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) oacc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
  }

  // Staging: piece i of a tile is token (tid + 256 i) / PIECES; a wave's pieces of
  // one i lie in one 16-token sub-tile, so the descriptor is wave-uniform.
  const int n_tiles = (n_sub + 1) >> 1;
  u32x4 gk[PER_T], gv[PER_T];
  auto gload = [&](int k) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int pc = tid + i * kWaves * 64;
      const int tok = pc / PIECES, piece = pc - tok * PIECES;
      const int u = 2 * k + (tok >> 4);
      int pb = 0, row0 = 0, nv = 0;
      if (u < n_sub) desc(u, pb, row0, nv);
      const size_t base = (size_t)pb * (size_t)c.block_bytes + (size_t)row0 * c.row_bytes;
      const unsigned off = (unsigned)((tok & 15) * c.row_bytes + g * D * 2 + piece * 16);
      gk[i] = buf_load16<0>(make_rsrc(c.kc + base, (unsigned)(nv * c.row_bytes)), off);
      gv[i] = buf_load16<0>(make_rsrc(c.vc + base, (unsigned)(nv * c.row_bytes)), off);
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* kb = s_kv + buf * 2 * TILEB;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int pc = tid + i * kWaves * 64;
      const int tok = pc / PIECES, piece = pc - tok * PIECES;
      *(u32x4*)(kb + tok * ROWB + piece * 16) = gk[i];
      *(u32x4*)(kb + TILEB + tok * ROWB + piece * 16) = gv[i];
    }
  };

  if (n_tiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int k = 0; k < n_tiles; ++k) {
    const bool more = k + 1 < n_tiles;
    if (more) gload(k + 1);
    if (active) {
      const unsigned char* kb = s_kv + (k & 1) * 2 * TILEB;
      const unsigned char* vb = kb + TILEB;
      int nv[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        int pb, row0;
        nv[sub] = 0;
        if (2 * k + sub < n_sub) desc(2 * k + sub, pb, row0, nv[sub]);
      }
      f32x4 sacc[RT][2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        u32x4 kf[KSTEPS];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
          kf[s] = *(const u32x4*)(kb + (16 * sub + r) * ROWB + (32 * s + 8 * qd) * 2);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          sacc[t][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) sacc[t][sub] = mfma16x16x32(kf[s], qf[t][s], sacc[t][sub]);
        }
      }
      u32x4 phi[RT], plo[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        float sv[8];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = sacc[t][sub][i] * c.qk_scale_log2;
            const bool ok = 4 * qd + i < nv[sub] &&
                            pos0 + 16 * (2 * k + sub) + 4 * qd + i < rows.limit[t];
            sv[sub * 4 + i] = ok ? x : -INFINITY;
          }
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
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
      // V rows 4 qd + i of each sub-tile, channels CPL r .. (as the global-load layout).
      vvec vf[2][4];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vf[sub][i] = *(const vvec*)(vb + (16 * sub + 4 * qd + i) * ROWB + r * CPL * 2);
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
    }
    if (more) lstore((k + 1) & 1);
    __syncthreads();
  }

#pragma unroll
  for (int t = 0; t < RT; ++t) {
    float l_tot = l_run[t] + __shfl_xor(l_run[t], 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (r < rows.n_rows[t]) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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

__device__ __forceinline__ int clamp_ctx(int v, int max_ctx) {
  return v < 0 ? 0 : (v > max_ctx ? max_ctx : v);
}

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
  const int ctx = clamp_ctx(p.ctx[b], p.max_ctx);
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
  int* prefix;               // [B + 1] sub-tile prefix sums, written by workgroup 0
  const int* block_tables;
  const int* ctx;
  const int* topk;           // [B, H_kv, K] logical block ids (sparse only)
  long long NB;
  int B, max_blocks, max_ctx, nwg, topk_blocks;
};

// Exclusive prefix sum over the workgroup's 256 threads; *total gets the sum.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* s_wave, int* total) {
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
  for (int w = 0; w < kWaves; ++w) {
    const int x = s_wave[w];
    off += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// Work of a sequence, in 16-token sub-tiles: dense, its context; sparse,
// min(K, blocks) blocks. Valid ids of one KV head's list are distinct blocks of the
// sequence, so no head has more valid entries than that, wherever they sit in its
// list; lists from Top-K have exactly that many.
template <int D, bool SPARSE, bool FP8>
__global__ __launch_bounds__(kWaves * 64) void attn_balanced_kernel(const BalParams p) {
  __shared__ int s_pref[kMaxBalBatch + 1];
  __shared__ int s_pb[kBalTab];                  // physical block per table entry (-1: none)
  __shared__ int s_tok0[SPARSE ? kBalTab : 1];   // sparse: logical position of its row 0
  __shared__ int s_wave[kWaves];
  const int wg = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int B = p.B, bs = p.c.bs, Hkv = p.c.Hkv, G = p.c.G;
  const int spb = bs >> 4;   // sub-tiles per block

  // Sub-tile counts of every sequence, and their prefix sums (all workgroups
  // compute the same values; workgroup 0 also hands them to the combine).
  int carry = 0;
  for (int base = 0; base < B; base += kWaves * 64) {
    const int bb = base + tid;
    int n = 0;
    if (bb < B) {
      const int ctx = clamp_ctx(p.ctx[bb], p.max_ctx);
      if (SPARSE) {
        const int nb = (ctx + bs - 1) / bs;
        n = (nb < p.topk_blocks ? nb : p.topk_blocks) * spb;
      } else {
        n = (ctx + 15) >> 4;
      }
    }
    int tot;
    const int ex = wg_exclusive_scan(n, s_wave, &tot);
    if (bb < B) s_pref[bb + 1] = carry + ex + n;
    carry += tot;
  }
  if (tid == 0) s_pref[0] = 0;
  __syncthreads();
  if (wg == 0)
    for (int i = tid; i <= B; i += kWaves * 64) p.prefix[i] = s_pref[i];
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
    const int ub = (s0 > s_pref[b] ? s0 : s_pref[b]) - s_pref[b];
    const int ue = (s1 < s_pref[b + 1] ? s1 : s_pref[b + 1]) - s_pref[b];
    if (ue <= ub) continue;  // empty sequence
    const int ctx = clamp_ctx(p.ctx[b], p.max_ctx);
    const int nb = (ctx + bs - 1) / bs;
    // Table entries (blocks) the share touches: dense, logical blocks e0 ..;
    // sparse, positions e0 .. of each KV head's list with the invalid ids removed.
    const int e0 = ub / spb;
    const int n_ent = (ue - 1) / spb - e0 + 1;
    __syncthreads();  // the previous sequence's table is no longer read
    if (!SPARSE) {
      for (int e = tid; e < n_ent; e += kWaves * 64) {
        const int lb = e0 + e;
        const int pb = lb < nb ? p.block_tables[(size_t)b * p.max_blocks + lb] : -1;
        s_pb[e] = (pb >= 0 && pb < p.NB) ? pb : -1;
      }
    } else {
      for (int i = tid; i < Hkv * n_ent; i += kWaves * 64) s_pb[i] = -1;
      __syncthreads();
      // Compaction of each head's list, 64 entries per step: a valid entry's
      // position is the number of valid entries before it.
      for (int g = wave; g < Hkv; g += kWaves) {
        const int* lst = p.topk + ((size_t)b * Hkv + g) * p.topk_blocks;
        int run = 0;
        for (int c0 = 0; c0 < p.topk_blocks && run < e0 + n_ent; c0 += 64) {
          const int e = c0 + lane;
          const int id = e < p.topk_blocks ? lst[e] : -1;
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
    __syncthreads();
    const size_t slot = (size_t)wg + b;
    for (int g = wave; g < Hkv; g += kWaves) {
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
__global__ __launch_bounds__(kWaves * 64) void attn_sparse_direct_kernel(const DirectParams p) {
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
// Quest decode in one launch: block selection, then attention over the selection
// ---------------------------------------------------------------------------

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
};

template <int D>
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

  // Selection (as quest_select_fused_kernel, into LDS).
  for (int lb = tid; lb < nb; lb += kFusedThreads) s_pb[lb] = sp.bt[(size_t)b * sp.max_blocks + lb];
  const bool all = K >= nb;
  if (!all) stage_query<D>(sp, b, g * G, G, s_q);
  __syncthreads();
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
      score_blocks<D, kFusedUnroll>(sp, g, nb, lb0, [&](int lb) { return s_pb[lb]; }, s_pos, s_neg,
                                    [&](int lb, unsigned long long key) { s_key[lb] = key; });
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
  attend_head<D, false, false, 1>(p.c, g, ue > ub ? ue - ub : 0, desc, 0, rows);
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
  const int* ctx;           // split path
  const int* prefix;        // balanced path
  int Hq, Hkv, G, max_ctx, num_splits, split_tokens, sparse, balanced, B, nwg;
};

constexpr int kCombineThreads = 256;

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
    const long long pre0 = p.prefix[b];
    const long long pre1 = p.prefix[b + 1];
    r.S = p.prefix[p.B];
    if (pre1 <= pre0) {
      r.u_begin = r.u_end = 0;
    } else {
      r.u_begin = (int)(((pre0 + 1) * p.nwg - 1) / r.S);  // workgroup holding sub-tile pre0
      r.u_end = (int)((pre1 * p.nwg - 1) / r.S) + 1;      // ... and sub-tile pre1 - 1
    }
    r.lstride = (size_t)p.Hkv * G;
    r.ostride = r.lstride * D;
    r.lse0 = p.part_lse + ((size_t)b * p.Hkv + g) * G + hl;
    r.o0 = p.part_o + (((size_t)b * p.Hkv + g) * G + hl) * D;
  } else {
    const int ctx = p.ctx[b] < 0 ? 0 : (p.ctx[b] > p.max_ctx ? p.max_ctx : p.ctx[b]);
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
// merges that head's units on its own, without barriers.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_heads_kernel(const CombineParams p) {
  constexpr int TPU = D / 4;
  constexpr int SLOTS = kCombineThreads / TPU;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int slot = tid / TPU, c4 = tid % TPU;
  for (int hl = slot; hl < p.G; hl += SLOTS) {
    const UnitRange r = unit_range<D>(p, b, g, hl);
    float M = -INFINITY;
    for (int u = r.u_begin; u < r.u_end; ++u)
      if (r.live(u)) M = fmaxf(M, r.lse0[(size_t)u * r.lstride]);
    const float Mr = (M == -INFINITY) ? 0.f : M;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    int u = r.u_begin;
    for (; u + 3 < r.u_end; u += 4) {
      float l[4];
      f32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool ok = r.live(u + k);
        l[k] = ok ? r.lse0[(size_t)(u + k) * r.lstride] : -INFINITY;
        v[k] = ok ? *(const f32x4*)(r.o0 + (size_t)(u + k) * r.ostride + 4 * c4)
                  : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = __builtin_amdgcn_exp2f(l[k] - Mr);
        W += w;
        acc += w * v[k];
      }
    }
    for (; u < r.u_end; ++u) {
      if (!r.live(u)) continue;
      const float w = __builtin_amdgcn_exp2f(r.lse0[(size_t)u * r.lstride] - Mr);
      W += w;
      acc += w * *(const f32x4*)(r.o0 + (size_t)u * r.ostride + 4 * c4);
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    *(f32x4*)(p.out + ((size_t)b * p.Hq + (size_t)g * p.G + hl) * D + 4 * c4) = acc * inv;
  }
}

template <int D>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(const CombineParams p) {
  constexpr int TPU = D / 4;                       // threads per unit row
  constexpr int UPP = kCombineThreads / TPU;       // units per pass
  __shared__ float s_red[kCombineThreads];
  __shared__ f32x4 s_acc[UPP][TPU];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int G = p.G;
  const int g = h / G, hl = h - g * G;
  float* out = p.out + ((size_t)b * p.Hq + h) * D;

  const UnitRange r = unit_range<D>(p, b, g, hl);
  if (r.u_end <= r.u_begin) {
    for (int c = tid; c < D; c += kCombineThreads) out[c] = 0.f;
    return;
  }
  const int u_begin = r.u_begin, u_end = r.u_end;
  const float* lse0 = r.lse0;
  const float* o0 = r.o0;
  const size_t lstride = r.lstride, ostride = r.ostride;
  auto live = [&](int u) { return r.live(u); };

  // Common maximum of the units' lse.
  const int lane = tid & 63, wave = tid >> 6;
  float M = -INFINITY;
  for (int u = u_begin + tid; u < u_end; u += kCombineThreads)
    if (live(u)) M = fmaxf(M, lse0[(size_t)u * lstride]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float Mr = (M == -INFINITY) ? 0.f : M;

  // Weighted sum: thread (unit slot us, float4 column c4) walks units us, us+UPP,
  // ..., eight loads in flight at a time.
  constexpr int UNROLL = 8;
  const int us = tid / TPU, c4 = tid % TPU;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  int u = u_begin + us;
  for (; u + (UNROLL - 1) * UPP < u_end; u += UNROLL * UPP) {
    float l[UNROLL];
    f32x4 v[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const int uu = u + k * UPP;
      const bool ok = live(uu);
      l[k] = ok ? lse0[(size_t)uu * lstride] : -INFINITY;
      v[k] = ok ? *(const f32x4*)(o0 + (size_t)uu * ostride + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const float w = __builtin_amdgcn_exp2f(l[k] - Mr);
      W += w;
      acc += w * v[k];
    }
  }
  for (; u < u_end; u += UPP) {
    if (!live(u)) continue;
    const float w = __builtin_amdgcn_exp2f(lse0[(size_t)u * lstride] - Mr);
    W += w;
    acc += w * *(const f32x4*)(o0 + (size_t)u * ostride + 4 * c4);
  }
  __syncthreads();  // s_red is reused below
  s_acc[us][c4] = acc;
  if (c4 == 0) s_red[us] = W;
  __syncthreads();
  if (tid < TPU) {
    f32x4 a = s_acc[0][tid];
    float wt = s_red[0];
#pragma unroll
    for (int k = 1; k < UPP; ++k) {
      a += s_acc[k][tid];
      wt += s_red[k];
    }
    const float inv = wt > 0.f ? 1.f / wt : 0.f;
    *(f32x4*)(out + 4 * tid) = a * inv;
  }
}

// ---------------------------------------------------------------------------
// Multi-token queries (varlen): rows = (query token, head) pairs, causal mask
// aligned to the right ([TL18] 2.7, 3.3)
// ---------------------------------------------------------------------------
//
// Query row m of sequence b's chunk (m < q_len * G) is token j = m / G, head
// g * G + m % G; a 16-row tile of these rows is one MFMA row block, so a chunk
// of q_len tokens costs ceil(q_len * G / 16) passes over the KV it sees (one pass
// for decode-sized chunks: q_len * G <= 16). Row j sees positions
// t <= ctx - q_len + j. Grid (row tile, split, sequence): the row tiles of one
// KV split are neighbours in launch order, so they read that split together.

struct VarlenParams {
  AttnCommon c;
  float* part_o;             // [tiles, H_kv, S, 16, D] fp32 (tile = tile_base(b) + rt)
  float* part_lse;           // [tiles, H_kv, S, 16] fp32 (base 2)
  float* out;                // [total_q, H_q, D] fp32 (combine)
  const int* block_tables;
  const int* ctx;
  const int* cu;             // [B + 1] query row offsets
  long long NB;
  int max_blocks, max_ctx, num_splits, split_tokens, n_rt, total_q, B;
};

// Partial rows of sequence b's row tiles sit at tiles tile_base(b) + rt: the
// (token, head) rows of the whole batch in 16-row steps, plus one per sequence
// for its partial last tile -- disjoint, and fewer than ceil(total_q * G / 16) + B.
__device__ __forceinline__ size_t tile_base(int q0, int G, int b) {
  return ((size_t)q0 * G) / 16 + (size_t)b;
}

// A sequence's query rows, with bad offsets (outside [0, total_q] or decreasing)
// read as an empty chunk so that no row outside the query buffer is touched.
__device__ __forceinline__ void varlen_rows(const VarlenParams& p, int b, int& q0, int& qn) {
  q0 = p.cu[b];
  const int q1 = p.cu[b + 1];
  if (q0 < 0 || q1 < q0 || q1 > p.total_q) {
    q0 = 0;
    qn = 0;
  } else {
    qn = q1 - q0;
  }
}

// Prefix over the sequences of per-sequence counts n(b) into s_pref[0..B] (every
// thread of the workgroup calls it; B <= kMaxBalBatch). Returns the total.
template <class Count>
__device__ __forceinline__ int sequence_prefix(int B, int* s_pref, int* s_wave, const Count& count) {
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < B; base += kWaves * 64) {
    const int bb = base + tid;
    const int n = bb < B ? count(bb) : 0;
    int tot;
    const int ex = wg_exclusive_scan(n, s_wave, &tot);
    if (bb < B) s_pref[bb + 1] = carry + ex + n;
    carry += tot;
  }
  if (tid == 0) s_pref[0] = 0;
  __syncthreads();
  return s_pref[B];
}

// The last b with s_pref[b] <= u (u < s_pref[B]).
__device__ __forceinline__ int sequence_of(const int* s_pref, int B, int u) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pref[mid] <= u)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Work units of multi-token queries: (sequence, group of RT row tiles, KV split),
// split-major within a sequence so that the units running together read the
// same split; a unit's waves take the KV heads. Sequences with kShareMinTiles row
// tiles or more (chunks, RT > 1) instead take units of (sequence, KV head, group
// of kShareTiles row tiles, split): the four waves share that head's K / V through
// LDS (attend_shared). A fixed grid takes the units grid-stride: no workgroup is
// launched for a sequence's missing row tiles. Two waves per SIMD (at most 256
// registers) let one wave's MFMA work hide the other's loads; RT = 2 fits without
// spilling at D = 128.
constexpr int kShareTiles = 2 * kWaves;   // row tiles of one shared unit
constexpr int kShareMinTiles = 4;

template <int D, int RT, bool FP8>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(RT == 1 ? 3 : 2))) void attn_varlen_kernel(const VarlenParams p) {
  constexpr bool kShared = RT > 1 && !FP8;   // E4M3 caches: per-head units only
  __shared__ int s_pb[kMaxTable];
  __shared__ int s_pref[kMaxBalBatch + 1];
  __shared__ int s_wave[kWaves];
  __shared__ __align__(16) unsigned char s_kv[kShared ? kShareLdsBytes(D) : 16];
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int bs = p.c.bs, Hkv = p.c.Hkv, G = p.c.G;
  const int T = p.split_tokens;
  auto n_tiles_of = [&](int qn) { return (qn * G + 15) / 16; };
  auto n_groups = [&](int qn) { return (n_tiles_of(qn) + RT - 1) / RT; };
  auto shared_seq = [&](int qn) { return kShared && n_tiles_of(qn) >= kShareMinTiles; };
  const int U = sequence_prefix(p.B, s_pref, s_wave, [&](int b) {
    const int ctx = clamp_ctx(p.ctx[b], p.max_ctx);
    int q0, qn;
    varlen_rows(p, b, q0, qn);
    if (qn <= 0 || ctx <= 0) return 0;
    const int ns = (ctx + T - 1) / T;
    return shared_seq(qn) ? (n_tiles_of(qn) + kShareTiles - 1) / kShareTiles * Hkv * ns
                          : n_groups(qn) * ns;
  });
  const int r = tid & 15;
  for (int u = blockIdx.x; u < U; u += gridDim.x) {
    const int b = sequence_of(s_pref, p.B, u);
    const int ctx = clamp_ctx(p.ctx[b], p.max_ctx);
    int q0, qn;
    varlen_rows(p, b, q0, qn);
    const int rows = qn * G;
    const int local = u - s_pref[b];
    const bool shared = shared_seq(qn);
    int split, g_sh = 0, m_first, m_span;
    if (shared) {
      const int n_grp = (n_tiles_of(qn) + kShareTiles - 1) / kShareTiles;
      const int grp = local % n_grp, rest = local / n_grp;
      g_sh = rest % Hkv;
      split = rest / Hkv;
      m_first = 16 * kShareTiles * grp;
      m_span = 16 * kShareTiles;
    } else {
      const int ntg = n_groups(qn);
      split = local / ntg;
      m_first = 16 * RT * (local % ntg);
      m_span = 16 * RT;
    }
    // Positions the unit's last row sees (the others see fewer).
    const int m_last = (m_first + m_span < rows ? m_first + m_span : rows) - 1;
    int tile_lim = ctx - qn + m_last / G + 1;
    tile_lim = tile_lim < 0 ? 0 : (tile_lim > ctx ? ctx : tile_lim);
    const int t0 = split * T;
    if (t0 >= tile_lim) continue;   // uniform: the combine counts only the splits a tile sees
    const int e0 = t0 / bs;
    const int n_ent = T / bs;
    const int nb = (ctx + bs - 1) / bs;
    __syncthreads();                // the previous unit's table is no longer read
    for (int e = tid; e < n_ent; e += kWaves * 64) {
      const int lb = e0 + e;
      const int pb = lb < nb ? p.block_tables[(size_t)b * p.max_blocks + lb] : -1;
      s_pb[e] = (pb >= 0 && pb < p.NB) ? pb : -1;
    }
    __syncthreads();
    const int span = tile_lim - t0 < T ? tile_lim - t0 : T;
    auto desc = [&](int uu, int& pb, int& row0, int& nv) {
      const int tok = t0 + 16 * uu;
      const int x = s_pb[tok / bs - e0];
      row0 = tok & (bs - 1);
      int n = t0 + span - tok;
      n = n < 0 ? 0 : (n > 16 ? 16 : n);
      if (x < 0) n = 0;
      nv = uniform(n);
      pb = uniform(x < 0 ? 0 : x);
    };
    // Row tile rt of the sequence against KV head g, as slot t of a RowTiles.
    auto fill = [&](auto& tiles, int t, int rt, int g) {
      const int m0 = 16 * rt;
      const int n_rows = rows - m0 < 0 ? 0 : (rows - m0 < 16 ? rows - m0 : 16);
      const int m = m0 + r, j = m / G;
      tiles.q[t] = r < n_rows
                       ? p.c.q + ((size_t)(q0 + j) * p.c.Hq + (size_t)g * G + (m - j * G)) * D
                       : nullptr;
      tiles.n_rows[t] = n_rows;
      tiles.limit[t] = ctx - qn + j + 1;
      const size_t unit =
          ((tile_base(q0, G, b) + (n_rows > 0 ? rt : 0)) * Hkv + g) * p.num_splits + split;
      tiles.o[t] = p.part_o + unit * 16 * D;
      tiles.lse[t] = p.part_lse + unit * 16;
    };
    if constexpr (kShared) {
      if (shared) {
        RowTiles<2> tiles;
        fill(tiles, 0, m_first / 16 + 2 * wave, g_sh);
        fill(tiles, 1, m_first / 16 + 2 * wave + 1, g_sh);
        attend_shared<D>(p.c, g_sh, (span + 15) / 16, desc, t0, tiles, s_kv);
        continue;
      }
    }
    for (int g = wave; g < Hkv; g += kWaves) {
      RowTiles<RT> tiles;
#pragma unroll
      for (int t = 0; t < RT; ++t) fill(tiles, t, m_first / 16 + t, g);
      attend_head<D, FP8, true, RT>(p.c, g, (span + 15) / 16, desc, t0, tiles);
    }
  }
}

// Merge of each (sequence, row tile, KV head) over its splits, written to the
// flattened output rows; the triples taken grid-stride.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void attn_varlen_combine_kernel(const VarlenParams p) {
  __shared__ int s_pref[kMaxBalBatch + 1];
  __shared__ int s_wave[kWaves];
  constexpr int TPR = D / 4;   // threads per row, 4 channels each
  const int G = p.c.G, Hq = p.c.Hq, Hkv = p.c.Hkv;
  const int U = sequence_prefix(p.B, s_pref, s_wave, [&](int b) {
    int q0, qn;
    varlen_rows(p, b, q0, qn);
    return (qn * G + 15) / 16 * Hkv;
  });
  for (int u = blockIdx.x; u < U; u += gridDim.x) {
    const int b = sequence_of(s_pref, p.B, u);
    const int local = u - s_pref[b];
    const int rt = local / Hkv, g = local - (local / Hkv) * Hkv;
    const int ctx = clamp_ctx(p.ctx[b], p.max_ctx);
    int q0, qn;
    varlen_rows(p, b, q0, qn);
    const int rows = qn * G;
    const int m0 = 16 * rt;
    const int n_rows = rows - m0 < 16 ? rows - m0 : 16;
    int tile_lim = ctx - qn + (m0 + n_rows - 1) / G + 1;
    tile_lim = tile_lim < 0 ? 0 : (tile_lim > ctx ? ctx : tile_lim);
    const int n_units = (tile_lim + p.split_tokens - 1) / p.split_tokens;
    const size_t unit0 = ((tile_base(q0, G, b) + rt) * Hkv + g) * p.num_splits;
    for (int i = threadIdx.x; i < n_rows * TPR; i += kCombineThreads) {
      const int rr = i / TPR, c4 = i - (i / TPR) * TPR;
      const float* lse0 = p.part_lse + unit0 * 16 + rr;
      const float* o0 = p.part_o + (unit0 * 16 + rr) * D + 4 * c4;
      float M = -INFINITY;
      for (int k = 0; k < n_units; ++k) M = fmaxf(M, lse0[(size_t)k * 16]);
      const float Mr = (M == -INFINITY) ? 0.f : M;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      float W = 0.f;
      int k = 0;
      for (; k + 3 < n_units; k += 4) {   // four splits' rows in flight
        float l[4];
        f32x4 v[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          l[x] = lse0[(size_t)(k + x) * 16];
          v[x] = *(const f32x4*)(o0 + (size_t)(k + x) * 16 * D);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float w = __builtin_amdgcn_exp2f(l[x] - Mr);
          W += w;
          acc += w * v[x];
        }
      }
      for (; k < n_units; ++k) {
        const float w = __builtin_amdgcn_exp2f(lse0[(size_t)k * 16] - Mr);
        W += w;
        acc += w * *(const f32x4*)(o0 + (size_t)k * 16 * D);
      }
      const float inv = W > 0.f ? 1.f / W : 0.f;
      const int m = m0 + rr, j = m / G;
      *(f32x4*)(p.out + ((size_t)(q0 + j) * Hq + (size_t)g * G + (m - j * G)) * D + 4 * c4) =
          acc * inv;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups of the balanced kernel: one per compute unit. Measured on MI355X
// over an 8K-average ragged batch: one 4-wave workgroup per CU streams the KV
// cache at ~6.1 TB/s, while two or three per CU (all resident) reach only 5.7
// and 5.4 TB/s, and counts that are not a multiple of the CU count (192, 320,
// 384) leave some CUs with two shares. One wave per SIMD, each with a 32-token
// tile in flight, already covers HBM latency; more concurrent streams only add
// DRAM conflicts.
static int balanced_capacity() {
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
    long long n = balanced_capacity();
    const long long need = (max_sub + share_max - 1) / share_max;
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

template <int D, bool SPARSE, bool FP8>
static void launch_attention(bool balanced, const BalParams& bp, const SplitParams& sp, int nwg,
                             int num_splits, int B, hipStream_t stream) {
  const dim3 block(kWaves * 64);
  if (balanced)
    attn_balanced_kernel<D, SPARSE, FP8><<<dim3(nwg), block, 0, stream>>>(bp);
  else
    attn_split_kernel<D, SPARSE, FP8><<<dim3(num_splits, B), block, 0, stream>>>(sp);
}

static int attn_run(bool sparse, bool fp8, float* out, const void* query, const void* kc,
                    const void* vc, const float* k_scale, const float* v_scale, const int* bt,
                    const int* ctx, const int* topk, int B, int Hq, int Hkv, int D, int bs,
                    long long NB, int max_blocks, int max_ctx, int K, float scale, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  const char* fn = sparse ? (fp8 ? "sparse_paged_attention_decode_fp8" : "sparse_paged_attention_decode")
                          : (fp8 ? "paged_attention_decode_fp8" : "paged_attention_decode");
  int st = check_common(fn, B, Hq, Hkv, D, bs, NB, max_blocks, max_ctx);
  if (st) return st;
  if (sparse && K < 1) return fail(GPKV_ERR_SHAPE, "%s: topk_blocks=%d < 1", fn, K);
  if (B == 0) return GPKV_OK;
  if (!out || !query || !kc || !vc || !bt || !ctx || (sparse && !topk) ||
      (fp8 && (!k_scale || !v_scale)))
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
  // Many units per sequence (long sequences over many workgroups or splits): one
  // workgroup per query head, its threads spread over the units. Few units: one
  // workgroup per KV head, a slot of threads per query head.
  const long long units_per_seq = pl.balanced ? (long long)pl.nwg / B + 1 : pl.num_splits;
  const dim3 cblock(kCombineThreads);
  if (units_per_seq >= 6) {
    const dim3 cgrid(Hq, B);
    if (D == 128)
      attn_combine_kernel<128><<<cgrid, cblock, 0, stream>>>(cp);
    else
      attn_combine_kernel<64><<<cgrid, cblock, 0, stream>>>(cp);
  } else {
    const dim3 cgrid(Hkv, B);
    if (D == 128)
      attn_combine_heads_kernel<128><<<cgrid, cblock, 0, stream>>>(cp);
    else
      attn_combine_heads_kernel<64><<<cgrid, cblock, 0, stream>>>(cp);
  }
  return check_launch(fn);
}

// Multi-token queries: row tiles per sequence, split size and workspace.
constexpr long long kVarlenMaxUnits = 1LL << 18;   // partial-row blocks (about 2 GB at D = 128)
constexpr int kVarlenRT = 2;   // row tiles per wave when a chunk spans more than one tile

struct VarlenPlan {
  int n_rt, split_tokens, num_splits;
  size_t o_bytes, lse_bytes;
};

// Row tiles of the longest chunk (the grid), split size, and the workspace for at
// most ceil(total_q * G / 16) + B row tiles. Decode-sized chunks split the KV like
// decode; longer chunks keep splits short (512 positions) so that no workgroup
// walks a long KV range alone.
static VarlenPlan make_varlen_plan(int B, int total_q, int max_q_len, int Hq, int Hkv, int D,
                                   int bs, int max_ctx) {
  VarlenPlan pl;
  const long long G = Hq / Hkv;
  const long long n_rt = (max_q_len * G + 15) / 16;
  pl.n_rt = (int)(n_rt > 0 ? n_rt : 1);
  const long long tiles = ((long long)total_q * G + 15) / 16 + B;
  // Multi-token chunks: long splits keep each group of row tiles on its tile loop and
  // cut the partial rows the combine reads (2048 measured best for mixed batches of
  // 8K-token contexts); one-token rows use the decode heuristic.
  const int forced = env_split_tokens();
  int T = forced ? forced : (pl.n_rt > 1 ? 2048 : split_tokens_for(B, Hkv, max_ctx));
  auto units = [&](int t) {
    const long long ns = ((long long)max_ctx + t - 1) / t;
    return tiles * Hkv * (ns > 0 ? ns : 1);
  };
  while (units(T) > kVarlenMaxUnits && T < 16384) T <<= 1;
  while (T / bs > kMaxTable) T >>= 1;
  pl.split_tokens = T;
  pl.num_splits = (int)(((long long)max_ctx + T - 1) / T);
  if (pl.num_splits < 1) pl.num_splits = 1;
  const size_t u = (size_t)tiles * Hkv * pl.num_splits;
  pl.o_bytes = align256(u * 16 * D * sizeof(float));
  pl.lse_bytes = align256(u * 16 * sizeof(float));
  return pl;
}

}  // namespace gpkv

using namespace gpkv;

extern "C" size_t gpkv_paged_attention_varlen_workspace_bytes(int32_t batch, int32_t total_q,
                                                              int32_t max_q_len,
                                                              int32_t num_q_heads,
                                                              int32_t num_kv_heads,
                                                              int32_t head_dim,
                                                              int32_t block_size,
                                                              int32_t max_context_len) {
  if (batch < 0 || total_q < 0 || max_q_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || !supported_head_dim(head_dim) ||
      !supported_block_size(block_size) || max_context_len < 0)
    return 0;
  const VarlenPlan pl = make_varlen_plan(batch, total_q, max_q_len, num_q_heads, num_kv_heads,
                                         head_dim, block_size, max_context_len);
  return pl.o_bytes + pl.lse_bytes;
}

template <bool FP8>
static void launch_varlen(bool multi, int head_dim, dim3 grid, dim3 block, hipStream_t s,
                          const VarlenParams& vp) {
  if (!multi) {
    if (head_dim == 128)
      attn_varlen_kernel<128, 1, FP8><<<grid, block, 0, s>>>(vp);
    else
      attn_varlen_kernel<64, 1, FP8><<<grid, block, 0, s>>>(vp);
  } else {
    if (head_dim == 128)
      attn_varlen_kernel<128, kVarlenRT, FP8><<<grid, block, 0, s>>>(vp);
    else
      attn_varlen_kernel<64, kVarlenRT, FP8><<<grid, block, 0, s>>>(vp);
  }
}

static int varlen_run(bool fp8, float* out, const void* query, const void* key_cache,
                      const void* value_cache, const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* cu_seqlens_q, int32_t batch, int32_t total_q,
                      int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                      int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = fp8 ? "paged_attention_varlen_fp8" : "paged_attention_varlen";
  int st = check_common(fn, batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_blocks_per_seq, max_context_len);
  if (st) return st;
  if (total_q < 0 || max_q_len < 0)
    return fail(GPKV_ERR_SHAPE, "%s: total_q=%d max_q_len=%d", fn, total_q, max_q_len);
  if (batch == 0 || total_q == 0) return GPKV_OK;
  if (max_q_len == 0) return fail(GPKV_ERR_SHAPE, "%s: max_q_len=0 with total_q=%d", fn, total_q);
  if (batch > kMaxBalBatch)
    return fail(GPKV_ERR_UNSUPPORTED, "%s: batch=%d > %d", fn, batch, kMaxBalBatch);
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !cu_seqlens_q || (fp8 && (!k_scale || !v_scale)))
    return fail(GPKV_ERR_NULL, "%s: null pointer argument", fn);
  const VarlenPlan pl = make_varlen_plan(batch, total_q, max_q_len, num_q_heads, num_kv_heads,
                                         head_dim, block_size, max_context_len);
  if (pl.num_splits > 65535)
    return fail(GPKV_ERR_SHAPE, "%s: max_context_len=%d needs too many splits", fn,
                max_context_len);
  const size_t need = pl.o_bytes + pl.lse_bytes;
  if (!workspace || workspace_bytes < need)
    return fail(GPKV_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  hipStream_t s = (hipStream_t)stream;
  VarlenParams vp;
  vp.c.q = (const unsigned short*)query;
  vp.c.kc = (const unsigned char*)key_cache;
  vp.c.vc = (const unsigned char*)value_cache;
  vp.c.k_scale = k_scale;
  vp.c.v_scale = v_scale;
  vp.c.row_bytes = num_kv_heads * head_dim * (fp8 ? 1 : 2);
  vp.c.block_bytes = (long long)block_size * vp.c.row_bytes;
  vp.c.Hq = num_q_heads;
  vp.c.Hkv = num_kv_heads;
  vp.c.G = num_q_heads / num_kv_heads;
  vp.c.bs = block_size;
  vp.c.qk_scale_log2 = scale * 1.4426950408889634f;
  vp.part_o = (float*)workspace;
  vp.part_lse = (float*)((char*)workspace + pl.o_bytes);
  vp.out = out;
  vp.block_tables = block_tables;
  vp.ctx = context_lens;
  vp.cu = cu_seqlens_q;
  vp.NB = num_blocks;
  vp.max_blocks = max_blocks_per_seq;
  vp.max_ctx = max_context_len;
  vp.num_splits = pl.num_splits;
  vp.split_tokens = pl.split_tokens;
  vp.n_rt = pl.n_rt;
  vp.total_q = total_q;
  vp.B = batch;
  // One row tile per wave for decode-sized chunks; otherwise kVarlenRT tiles share
  // every K / V tile a wave loads. Both kernels take their work units grid-stride
  // from a fixed grid of at most four workgroups per CU.
  const int rt_per_wave = pl.n_rt > 1 ? kVarlenRT : 1;
  const long long tiles = ((long long)total_q * vp.c.G + 15) / 16 + batch;
  const long long units_max = (tiles / rt_per_wave + batch) * pl.num_splits;
  const long long cap = 4LL * balanced_capacity();
  const dim3 grid((unsigned)(units_max < cap ? units_max : cap)), block(kWaves * 64);
  if (fp8)
    launch_varlen<true>(rt_per_wave > 1, head_dim, grid, block, s, vp);
  else
    launch_varlen<false>(rt_per_wave > 1, head_dim, grid, block, s, vp);
  st = check_launch(fn);
  if (st) return st;
  const long long ctiles = tiles * num_kv_heads;
  const dim3 cgrid((unsigned)(ctiles < cap ? ctiles : cap)), cblock(kCombineThreads);
  if (head_dim == 128)
    attn_varlen_combine_kernel<128><<<cgrid, cblock, 0, s>>>(vp);
  else
    attn_varlen_combine_kernel<64><<<cgrid, cblock, 0, s>>>(vp);
  return check_launch(fn);
}

extern "C" int gpkv_paged_attention_varlen(
    float* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_seqlens_q,
    int32_t batch, int32_t total_q, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return varlen_run(false, out, query, key_cache, value_cache, nullptr, nullptr, block_tables,
                    context_lens, cu_seqlens_q, batch, total_q, max_q_len, num_q_heads,
                    num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                    max_context_len, scale, workspace, workspace_bytes, stream);
}

extern "C" int gpkv_paged_attention_varlen_fp8(
    float* out, const void* query, const void* key_cache, const void* value_cache,
    const float* k_scale, const float* v_scale, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* cu_seqlens_q, int32_t batch, int32_t total_q,
    int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    float scale, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return varlen_run(true, out, query, key_cache, value_cache, k_scale, v_scale, block_tables,
                    context_lens, cu_seqlens_q, batch, total_q, max_q_len, num_q_heads,
                    num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                    max_context_len, scale, workspace, workspace_bytes, stream);
}

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

// One launch for the Quest decode step when the (sequence, KV head) pairs fill
// between half of the CUs and all of them (one 512-thread workgroup per CU: the
// attention's registers leave room for no second one); otherwise the selection
// and the sparse attention calls in turn, sharing the workspace.
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
  const char* fn = "quest_decode";
  int st = check_common(fn, batch, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_blocks_per_seq, max_context_len);
  if (st) return st;
  if (topk_blocks < 1) return fail(GPKV_ERR_SHAPE, "%s: topk_blocks=%d < 1", fn, topk_blocks);
  if ((long long)topk_blocks * block_size > (1LL << 30))
    return fail(GPKV_ERR_SHAPE, "%s: token span too large", fn);
  if (batch == 0) return GPKV_OK;
  if (!out || !topk_indices || !query || !key_cache || !value_cache || !key_min || !key_max ||
      !block_tables || !context_lens)
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
  bool fused = fits && 2 * pairs > cus && pairs <= cus;
  const char* forced = getenv("GPKV_QUEST_DECODE_PATH");
  if (forced && strcmp(forced, "fused") == 0) fused = fits;
  if (forced && strcmp(forced, "separate") == 0) fused = false;
  if (!fused) {
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
  sp.kmin = (const unsigned short*)key_min;
  sp.kmax = (const unsigned short*)key_max;
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
  c.k_scale = nullptr;
  c.v_scale = nullptr;
  c.row_bytes = num_kv_heads * head_dim * 2;
  c.block_bytes = (long long)block_size * c.row_bytes;
  c.Hq = num_q_heads;
  c.Hkv = num_kv_heads;
  c.G = G;
  c.bs = block_size;
  c.qk_scale_log2 = scale * 1.4426950408889634f;
  qp.out = out;
  qp.max_nb = max_nb;
  const dim3 grid(num_kv_heads, batch), block(kFusedThreads);
  hipStream_t s = (hipStream_t)stream;
  if (head_dim == 128)
    quest_decode_fused_kernel<128><<<grid, block, lds, s>>>(qp);
  else
    quest_decode_fused_kernel<64><<<grid, block, lds, s>>>(qp);
  return check_launch(fn);
}
