// Multi-token queries over the paged cache (varlen): rows = (query token, head)
// pairs, causal mask aligned to the right ([TL18] 2.7, 3.3), bf16 or E4M3 caches.
//
// Query row m of sequence b's chunk (m < q_len * G) is token j = m / G, head
// g * G + m % G; a 16-row tile of these rows is one MFMA row block, so a chunk
// of q_len tokens costs ceil(q_len * G / 16) passes over the KV it sees (one pass
// for decode-sized chunks: q_len * G <= 16). Row j sees positions
// t <= ctx - q_len + j. Grid (row tile, split, sequence): the row tiles of one
// KV split are neighbours in launch order, so they read that split together.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "attention.h"

namespace gpkv {

// Causal rows of one KV head shared by the whole workgroup: each wave carries two
// row tiles, and every 32-token K / V tile is loaded once per workgroup into LDS
// instead of once per wave. Same arithmetic as attend_head (S^T = K Q^T and
// O^T += V^T P^T on MFMA, P as a bf16 hi + lo pair); every wave of the workgroup
// must call it with the same n_sub, desc and pos0 (it has barriers). E4M3 caches
// (FP8): the staging threads load codes (half the bytes) and widen them to bf16
// (exact) as they store, so LDS holds the same bf16 tiles; K's scale joins the
// softmax scale and V's the final normalisation, as in attend_head.
//
// LDS holds two K and two V tiles:
//   - K token-major, rows padded to 2D + 16 bytes: lane (r, qd) reads token r's
//     channels 32s + 8qd .. +8 of k-step s as one 16-byte A operand;
//   - V channel-major as token pairs: row c (64 bytes) holds the 16 words
//     (V[2p][c], V[2p+1][c]), word p stored at position 4((p >> 1) & 3) + (p & 1) +
//     2(p >> 3), in 16-byte chunks whose index is XORed with (c >> 2) & 3. The
//     four words lane (r, qd) feeds to P.V tile j (channel 16j + r, contraction
//     slots 8qd .. +8: tokens 4qd .. +4 of sub-tile 0, then of sub-tile 1) are
//     then one aligned 16-byte chunk, and the 16 lanes of a row group hit
//     distinct banks. The staging threads do the transpose once per workgroup
//     instead of every wave repacking V with v_perm.
// Pipelining: tile k + 1's q.k MFMAs are issued before tile k's softmax, so the
// matrix cores work while the wave runs the softmax. K is staged two tiles ahead
// and V one tile ahead, double-buffered, one barrier per tile.
// Lazy rescale: the reference max of a row moves only when the tile's maximum
// exceeds it by more than kRescaleSlack (log2 units), so the weights stay below
// 2^kRescaleSlack and the rescale of O runs on few tiles; the result is the same
// softmax, normalised by the same reference.
constexpr int kShareKRowBytes(int D) { return 2 * D + 16; }
constexpr int kShareKTileBytes(int D) { return 32 * kShareKRowBytes(D); }
constexpr int kShareVTileBytes(int D) { return 64 * D; }
constexpr int kShareLdsBytes(int D) { return 2 * (kShareKTileBytes(D) + kShareVTileBytes(D)); }
constexpr float kRescaleSlack = 8.f;

// Maxima of raw MFMA results without the quieting of signalling NaNs that fmaxf
// adds in IEEE mode (one extra instruction per operand): a NaN score makes the
// row's output NaN either way.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_across_rows_raw(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_raw(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_raw(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

struct TileDesc {   // the two 16-token sub-tiles of one 32-token tile (wave-uniform)
  int pb[2], row0[2], nv[2];
};

template <int D, bool FP8, class Desc>
__device__ __forceinline__ void attend_shared(const AttnCommon& c, int g, int n_sub,
                                              const Desc& desc, int pos0, const RowTiles<2>& rows,
                                              unsigned char* s_kv) {
  constexpr int RT = 2;
  constexpr int KSTEPS = D / 32;
  constexpr int NJ = D / 16;                 // 16-channel tiles of O^T
  constexpr int KROWB = kShareKRowBytes(D);
  constexpr int KTILEB = kShareKTileBytes(D);
  constexpr int VTILEB = kShareVTileBytes(D);
  constexpr int KPIECES = 2 * D / 16;        // 16-byte pieces per K token row
  constexpr int K_PER_T = 32 * KPIECES / (kWaves * 64);   // K pieces per thread per tile
  static_assert(K_PER_T >= 1 && 32 * KPIECES == K_PER_T * kWaves * 64, "K tile split");
  constexpr int VPAIRS = D / 2;              // channel pairs: one V staging item per (chunk, pair)
  static_assert(4 * VPAIRS <= kWaves * 64, "V tile split");
  // V staging columns: channel pairs (bf16, 4 bytes per token) or channel quads (E4M3)
  constexpr int VCOLS = FP8 ? D / 4 : VPAIRS;
  constexpr int EB = FP8 ? 1 : 2;            // bytes per cached element
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = lane & 15, qd = lane >> 4;
  const bool active = rows.n_rows[0] > 0;   // the wave's second tile is empty if its first is
  // Causal bounds grow with the row, so row 0 of the first tile (lane 0) has the
  // smallest: a tile whose positions all lie below it, with every row of both
  // sub-tiles valid, needs no mask.
  const int lim_min = __builtin_amdgcn_readfirstlane(rows.limit[0]);
  // Scores are scaled inside the exponent's FMA, by |scale|; a negative scale
  // flips the sign of q instead (exact in bf16).
  float qks = c.qk_scale_log2;
  if constexpr (FP8) qks *= c.k_scale[g];
  const float scl = fabsf(qks);
  const unsigned qflip = qks < 0.f ? 0x80008000u : 0u;
  unsigned char* const kbuf = s_kv;
  unsigned char* const vbuf = s_kv + 2 * KTILEB;

  u32x4 qf[RT][KSTEPS];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[t][s] = rows.q[t] != nullptr
                     ? (*(const u32x4*)(rows.q[t] + 32 * s + 8 * qd)) ^ qflip
                     : u32x4{0u, 0u, 0u, 0u};
  }
  f32x4 oacc[RT][NJ];
  float m_run[RT], m_use[RT], l_run[RT];   // reference max (base 2), its finite stand-in, sum
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) oacc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[t] = -INFINITY;
    m_use[t] = 0.f;
    l_run[t] = 0.f;
  }

  const int n_tiles = (n_sub + 1) >> 1;
  // desc gives an empty sub-tile (nv = 0) past the span, so both sub-tiles are
  // described without a branch and their two table reads are in flight together.
  auto tdesc = [&](int k) {
    TileDesc d;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) desc(2 * k + sub, d.pb[sub], d.row0[sub], d.nv[sub]);
    return d;
  };
  // (sub is wave-uniform; selects rather than an indexed read keep TileDesc in
  // scalar registers)
  auto rsrc_of = [&](const unsigned char* cache, const TileDesc& d, int sub) {
    const int pb = sub ? d.pb[1] : d.pb[0], row0 = sub ? d.row0[1] : d.row0[0];
    const int nv = sub ? d.nv[1] : d.nv[0];
    const size_t base = (size_t)pb * (size_t)c.block_bytes + (size_t)row0 * c.row_bytes;
    return make_rsrc(cache + base, (unsigned)(nv * c.row_bytes));
  };
  // K staging: piece i of a thread is token (tid + 256 i) / KPIECES; a wave's
  // pieces of one i lie in one sub-tile, so the descriptor is wave-uniform.
  auto k_issue = [&](const TileDesc& d, u32x4 (&gk)[K_PER_T]) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int pc = tid + i * kWaves * 64;
      const int tok = pc / KPIECES, piece = pc - tok * KPIECES;
      // D = 128: piece i lies in sub-tile i; D = 64: waves 0-1 in sub-tile 0, 2-3 in 1.
      const int sub = K_PER_T > 1 ? i * 16 * KPIECES / (kWaves * 64) : uniform(tid >> 7);
      if constexpr (FP8) {   // the piece's 8 channels as 8 codes
        const unsigned off = (unsigned)((tok & 15) * c.row_bytes + g * D + piece * 8);
        const u32x2 x = buf_load8<0>(rsrc_of(c.kc, d, sub), off);
        gk[i] = u32x4{x[0], x[1], 0u, 0u};
      } else {
        const unsigned off = (unsigned)((tok & 15) * c.row_bytes + g * D * 2 + piece * 16);
        gk[i] = buf_load16<0>(rsrc_of(c.kc, d, sub), off);
      }
    }
  };
  auto k_store = [&](int buf, const u32x4 (&gk)[K_PER_T]) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int pc = tid + i * kWaves * 64;
      const int tok = pc / KPIECES, piece = pc - tok * KPIECES;
      u32x4 v = gk[i];
      if constexpr (FP8) {
        const u32x2 lo = e4m3x4_to_bf16(gk[i][0]), hi = e4m3x4_to_bf16(gk[i][1]);
        v = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      *(u32x4*)(kbuf + buf * KTILEB + tok * KROWB + piece * 16) = v;
    }
  };
  // V staging: item (chunk q, column cp) loads one word of tokens 4q .. 4q + 3 of
  // both sub-tiles -- channels 2cp, 2cp + 1 (bf16) or 4cp .. 4cp + 3 (E4M3 codes) --
  // and writes the chunk q of those channels' rows.
  const int v_item = tid < 4 * VCOLS ? tid : 0;
  const bool v_on = tid < 4 * VCOLS;
  const int vq = v_item / VCOLS, vcp = v_item - vq * VCOLS;
  auto v_issue = [&](const TileDesc& d, unsigned (&gv)[8]) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const __amdgpu_buffer_rsrc_t rv = rsrc_of(c.vc, d, sub);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        gv[4 * sub + i] = buf_load4<0>(rv, (unsigned)((4 * vq + i) * c.row_bytes + g * D * EB + vcp * 4));
    }
  };
  auto v_store = [&](int buf, const unsigned (&gv)[8]) {
    if (!v_on) return;
    if constexpr (FP8) {
      u32x2 cv[8];   // per token: channels (4cp, 4cp + 1) and (4cp + 2, 4cp + 3) as bf16 pairs
#pragma unroll
      for (int i = 0; i < 8; ++i) cv[i] = e4m3x4_to_bf16(gv[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 4 * vcp + e;
        u32x4 w;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
          w[dd] = (e & 1) ? pack_hi16(cv[2 * dd][e >> 1], cv[2 * dd + 1][e >> 1])
                          : pack_lo16(cv[2 * dd][e >> 1], cv[2 * dd + 1][e >> 1]);
        *(u32x4*)(vbuf + buf * VTILEB + ch * 64 + 16 * (vq ^ ((ch >> 2) & 3))) = w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int ch = 2 * vcp + e;
        u32x4 w;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
          w[dd] = e ? pack_hi16(gv[2 * dd], gv[2 * dd + 1]) : pack_lo16(gv[2 * dd], gv[2 * dd + 1]);
        *(u32x4*)(vbuf + buf * VTILEB + ch * 64 + 16 * (vq ^ ((ch >> 2) & 3))) = w;
      }
    }
  };
  // S^T of one tile (raw q.k) from K buffer kb.
  auto scores = [&](const unsigned char* kb, f32x4 (&sc)[RT][2]) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      u32x4 kf[KSTEPS];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        kf[s] = *(const u32x4*)(kb + (16 * sub + r) * KROWB + (32 * s + 8 * qd) * 2);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        sc[t][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) sc[t][sub] = mfma16x16x32(kf[s], qf[t][s], sc[t][sub]);
      }
    }
  };
  // Online softmax of tile k for row r of each row tile, then O^T += V^T P^T.
  // Masked scores become -inf in place, and only tiles that need a mask pay for it.
  auto softmax_pv = [&](int k, f32x4 (&sc)[RT][2], const TileDesc& d, const unsigned char* vb) {
    const bool full = d.nv[0] == 16 && d.nv[1] == 16 && pos0 + 32 * k + 32 <= lim_min;
    if (!full) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int bound = min(rows.limit[t] - (pos0 + 32 * k + 16 * sub), d.nv[sub]);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            if (4 * qd + ii >= bound) sc[t][sub][ii] = -INFINITY;
        }
    }
    u32x4 phi[RT], plo[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      float mx = max3_raw(max3_raw(sc[t][0][0], sc[t][0][1], sc[t][0][2]),
                          max3_raw(sc[t][0][3], sc[t][1][0], sc[t][1][1]),
                          max3_raw(sc[t][1][2], sc[t][1][3], -INFINITY));
      mx = max_across_rows_raw(mx);
      const float ms = mx == -INFINITY ? -INFINITY : mx * scl;   // the tile's scaled row max
      const bool up = ms > m_run[t] + kRescaleSlack;
      if (__any(up)) {
        const float m_new = up ? ms : m_run[t];
        const float alpha = up ? __builtin_amdgcn_exp2f(m_run[t] - m_new) : 1.f;   // 0 from -inf
#pragma unroll
        for (int j = 0; j < NJ; ++j) oacc[t][j] *= alpha;
        l_run[t] *= alpha;
        m_run[t] = m_new;
        m_use[t] = m_new == -INFINITY ? 0.f : m_new;
      }
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][i >> 2][i & 3], scl, -m_use[t]));
      if (!full) {   // exp2(-inf) is 0 already, unless |scale| = 0 made the FMA NaN
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = sc[t][i >> 2][i & 3] == -INFINITY ? 0.f : pv[i];
      }
      l_run[t] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const unsigned a = __float_as_uint(pv[2 * dd]), b = __float_as_uint(pv[2 * dd + 1]);
        phi[t][dd] = pack_hi16(a, b);
        const float ra = pv[2 * dd] - __uint_as_float(a & 0xffff0000u);
        const float rb = pv[2 * dd + 1] - __uint_as_float(b & 0xffff0000u);
        plo[t][dd] = pack_hi16(__float_as_uint(ra), __float_as_uint(rb));
      }
    }
    const unsigned vlane = (unsigned)(r * 64 + 16 * (qd ^ ((r >> 2) & 3)));
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const u32x4 va = *(const u32x4*)(vb + j * 1024 + vlane);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        oacc[t][j] = mfma16x16x32(va, phi[t], oacc[t][j]);
        oacc[t][j] = mfma16x16x32(va, plo[t], oacc[t][j]);
      }
    }
  };

  // Prologue: K and V of tile 0 and K of tile 1 in LDS, scores of tile 0.
  TileDesc d_cur = tdesc(0), d_next = tdesc(1);
  {
    u32x4 gk0[K_PER_T], gk1[K_PER_T];
    unsigned gv[8];
    k_issue(d_cur, gk0);
    v_issue(d_cur, gv);
    k_issue(d_next, gk1);
    k_store(0, gk0);
    v_store(0, gv);
    k_store(1, gk1);
  }
  __syncthreads();
  f32x4 sa[RT][2], sb[RT][2];
  if (active && n_tiles > 0) scores(kbuf, sa);
  __syncthreads();   // K buffer 0 is rewritten during tile 0

  // Tile k: stage K of k + 2 and V of k + 1 (loads issued for every tile, with
  // an empty descriptor past the end, so the wait counts are the same on every
  // path), scores of k + 1, softmax and P.V of k.
  auto step = [&](int k, f32x4 (&s_this)[RT][2], f32x4 (&s_next)[RT][2]) {
    const TileDesc d_nn = tdesc(k + 2);
    u32x4 gk[K_PER_T];
    unsigned gv[8];
    k_issue(d_nn, gk);
    v_issue(d_next, gv);
    if (active) {
      if (k + 1 < n_tiles) scores(kbuf + ((k + 1) & 1) * KTILEB, s_next);
      softmax_pv(k, s_this, d_cur, vbuf + (k & 1) * VTILEB);
    }
    k_store(k & 1, gk);
    v_store((k + 1) & 1, gv);
    __syncthreads();
    d_cur = d_next;
    d_next = d_nn;
  };
  for (int k = 0; k < n_tiles; k += 2) {
    step(k, sa, sb);
    if (k + 1 < n_tiles) step(k + 1, sb, sa);
  }

  float vsc = 1.f;
  if constexpr (FP8) vsc = c.v_scale[g];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const float l_tot = sum_across_rows(l_run[t]);
    if (r < rows.n_rows[t]) {
      const float inv = l_tot > 0.f ? vsc / l_tot : 0.f;
      float* dst = rows.o[t] + (size_t)r * D + 4 * qd;
#pragma unroll
      for (int j = 0; j < NJ; ++j) *(f32x4*)(dst + 16 * j) = oacc[t][j] * inv;
      if (qd == 0) rows.lse[t][r] = l_tot > 0.f ? m_run[t] + log2f(l_tot) : -INFINITY;
    }
  }
}

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
  int balanced;              // 1: balanced schedule (equal shares of the tile space)
  int slot_rows;             // balanced: row-tile rows per partial slot
  int nwg;                   // balanced: shares (a multiple of the split kernel's grid)
  int share_ok, rt;          // balanced: the split kernel's shared-LDS path and row tiles per wave
  int* unit_info;            // balanced: [units, 2] first workgroup covering a unit, and how many
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

constexpr int kShareTiles = 2 * kWaves;   // row tiles of one shared unit
constexpr int kShareMinTiles = 4;

// A sequence's work under the balanced schedule: groups of grp_rt row tiles (a
// shared group: one KV head per unit, so `heads` = H_kv units per group; a per-head
// group: one unit whose waves take the KV heads), each group's unit covering the
// 32-position tiles its last row sees. Units are ordered head-major, group minor.
struct SeqGeom {
  int ctx, q0, qn, rows, n_grp, grp_rt, heads;
  bool shared;
};

// share_ok: the launched kernel has the shared-LDS path; rt: its row tiles per wave.
__device__ __forceinline__ SeqGeom seq_geom(const VarlenParams& p, int b, bool share_ok, int rt) {
  SeqGeom sg;
  sg.ctx = clamp_ctx(p.ctx[b], p.max_ctx);
  varlen_rows(p, b, sg.q0, sg.qn);
  sg.rows = sg.qn * p.c.G;
  const int n_rt = (sg.rows + 15) / 16;
  sg.shared = share_ok && n_rt >= kShareMinTiles;
  sg.grp_rt = sg.shared ? kShareTiles : rt;
  sg.n_grp = (sg.qn > 0 && sg.ctx > 0) ? (n_rt + sg.grp_rt - 1) / sg.grp_rt : 0;
  sg.heads = sg.shared ? p.c.Hkv : 1;
  return sg;
}

// Positions the last row of group grp sees (the group's other rows see fewer).
__device__ __forceinline__ int group_limit(const SeqGeom& sg, int G, int grp) {
  int m_last = 16 * sg.grp_rt * (grp + 1);
  m_last = (m_last < sg.rows ? m_last : sg.rows) - 1;
  int lim = sg.ctx - sg.qn + m_last / G + 1;
  return lim < 0 ? 0 : (lim > sg.ctx ? sg.ctx : lim);
}
__device__ __forceinline__ int group_tiles(const SeqGeom& sg, int G, int grp) {
  return (group_limit(sg, G, grp) + 31) >> 5;
}
// Tiles of one head's units (every head of a shared sequence has the same).
__device__ __forceinline__ int head_tiles(const SeqGeom& sg, int G) {
  int t = 0;
  for (int grp = 0; grp < sg.n_grp; ++grp) t += group_tiles(sg, G, grp);
  return t;
}

// Work units of multi-token queries: (sequence, group of RT row tiles, KV split),
// split-major within a sequence so that the units running together read the
// same split; a unit's waves take the KV heads. Sequences with kShareMinTiles row
// tiles or more (chunks, RT > 1) instead take units of (sequence, KV head, group
// of kShareTiles row tiles, split): the four waves share that head's K / V through
// LDS (attend_shared). A fixed grid takes the units grid-stride: no workgroup is
// launched for a sequence's missing row tiles. At most 256 registers (two waves per
// SIMD): with row-tile pairs one wave's MFMA work hides the other's loads, and RT = 2
// fits without spilling at D = 128; single row tiles run one workgroup per CU.

// Balanced schedule: the flattened (unit, 32-position tile) space of the whole batch
// is shared out equally, [w*W/N, (w+1)*W/N) for workgroup w of N (all resident), so
// no workgroup waits for a last round. A workgroup runs the segments of the units
// its share touches; each segment writes its partial rows (normalised O, base-2
// lse) to slot w + (global index of the unit), unique because the shares are
// ordered; the combine merges the slots of the workgroups that covered a unit.
template <int D, int RT, bool FP8>
__device__ __forceinline__ void attn_varlen_balanced(const VarlenParams& p, int* s_pb, int* s_pref,
                                                     int* s_upref, int* s_wave,
                                                     unsigned char* s_kv) {
  constexpr bool kShared = RT > 1;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int bs = p.c.bs, Hkv = p.c.Hkv, G = p.c.G;
  const int bs_log2 = __builtin_ctz((unsigned)bs);
  const int r = tid & 15;
  auto geom = [&](int b) { return seq_geom(p, b, kShared, RT); };
  const int W = sequence_prefix(p.B, s_pref, s_wave, [&](int b) {
    const SeqGeom sg = geom(b);
    return sg.heads * head_tiles(sg, G);
  });
  sequence_prefix(p.B, s_upref, s_wave, [&](int b) {
    const SeqGeom sg = geom(b);
    return sg.heads * sg.n_grp;
  });
  // N shares, V consecutive ones per workgroup (N = V * grid): each share is short
  // enough for one staged table chunk, and every workgroup holds the same work.
  const int N = p.nwg, V = p.nwg / (int)gridDim.x;
  for (int w = (int)blockIdx.x * V; w < ((int)blockIdx.x + 1) * V; ++w) {
    const int s0 = (int)((long long)w * W / N), s1 = (int)((long long)(w + 1) * W / N);
    if (s0 >= s1) continue;
    int b = sequence_of(s_pref, p.B, s0);
    int pos = s0;
    while (pos < s1) {
      while (s_pref[b + 1] <= pos) ++b;   // skips sequences without work; pos < W
      const SeqGeom sg = geom(b);
      // The unit holding offset o: head h = o / (work per head), then its group.
      const int hw = head_tiles(sg, G);
      const int o = pos - s_pref[b];
      const int h = o / hw;
      int grp = 0, uoff = h * hw, wk = group_tiles(sg, G, 0);
      while (o >= uoff + wk) {
        uoff += wk;
        ++grp;
        wk = group_tiles(sg, G, grp);
      }
      const int ta = o - uoff;
      const int tb = (s1 - s_pref[b] - uoff < wk) ? s1 - s_pref[b] - uoff : wk;
      pos = s_pref[b] + uoff + tb;
      const int unit = s_upref[b] + h * sg.n_grp + grp;
      const int slot = w + unit;
      if (ta == 0 && tid == 0) {   // this share holds the unit's first tile: record its coverage
        const long long last = (((long long)s_pref[b] + uoff + wk) * N - 1) / W;
        p.unit_info[2 * unit] = w;
        p.unit_info[2 * unit + 1] = (int)(last - w + 1);
      }
      const int t0 = 32 * ta;
      const int lim = group_limit(sg, G, grp);
      const int span = (32 * (tb - ta) < lim - t0) ? 32 * (tb - ta) : lim - t0;
      const int e0 = t0 >> bs_log2;
      int n_ent = ((t0 + span - 1) >> bs_log2) - e0 + 1;
      n_ent = n_ent < kMaxTable ? n_ent : kMaxTable;   // the host sizes shares below this
      const int nb = (sg.ctx + bs - 1) / bs;
      __syncthreads();   // the previous segment's table is no longer read
      for (int e = tid; e < n_ent; e += kWaves * 64) {
        const int lb = e0 + e;
        const int pb = lb < nb ? p.block_tables[(size_t)b * p.max_blocks + lb] : -1;
        s_pb[e] = (pb >= 0 && pb < p.NB) ? pb : -1;
      }
      __syncthreads();
      auto desc = [&](int uu, int& pb, int& row0, int& nv) {
        const int tok = t0 + 16 * uu;
        const int ei = (tok >> bs_log2) - e0;
        const int xr = s_pb[ei < n_ent ? ei : 0];   // read unconditionally, in bounds
        const int x = ei < n_ent ? xr : -1;
        row0 = tok & (bs - 1);
        int n = t0 + span - tok;
        n = n < 0 ? 0 : (n > 16 ? 16 : n);
        if (x < 0) n = 0;
        nv = uniform(n);
        pb = uniform(x < 0 ? 0 : x);
      };
      // Row tile rt of the sequence against KV head g, into slot row srow.
      auto fill = [&](auto& tiles, int t, int rt, int g, int srow) {
        const int m0 = 16 * rt;
        const int n_rows = sg.rows - m0 < 0 ? 0 : (sg.rows - m0 < 16 ? sg.rows - m0 : 16);
        const int m = m0 + r, j = m / G;
        tiles.q[t] = r < n_rows
                         ? p.c.q + ((size_t)(sg.q0 + j) * p.c.Hq + (size_t)g * G + (m - j * G)) * D
                         : nullptr;
        tiles.n_rows[t] = n_rows;
        tiles.limit[t] = sg.ctx - sg.qn + j + 1;
        const size_t row_blk = (size_t)slot * p.slot_rows + srow;
        tiles.o[t] = p.part_o + row_blk * 16 * D;
        tiles.lse[t] = p.part_lse + row_blk * 16;
      };
      const int n_sub = (span + 15) / 16;
      if constexpr (kShared) {
        if (sg.shared) {
          RowTiles<2> tiles;
          const int rt0 = grp * kShareTiles + 2 * wave;
          fill(tiles, 0, rt0, h, 2 * wave);
          fill(tiles, 1, rt0 + 1, h, 2 * wave + 1);
          attend_shared<D, FP8>(p.c, h, n_sub, desc, t0, tiles, s_kv);
          continue;
        }
      }
      for (int g = wave; g < Hkv; g += kWaves) {
        RowTiles<RT> tiles;
  #pragma unroll
        for (int t = 0; t < RT; ++t) fill(tiles, t, grp * RT + t, g, g * RT + t);
        attend_head<D, FP8, true, RT>(p.c, g, n_sub, desc, t0, tiles);
      }
    }
  }
}

template <int D, int RT, bool FP8, bool BAL>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_varlen_kernel(const VarlenParams p) {
  constexpr bool kShared = RT > 1;
  __shared__ int s_pb[kMaxTable];
  __shared__ int s_pref[kMaxBalBatch + 1];
  __shared__ int s_upref[kMaxBalBatch + 1];   // balanced: unit prefix over sequences
  __shared__ int s_wave[kWaves];
  __shared__ __align__(16) unsigned char s_kv[kShared ? kShareLdsBytes(D) : 16];
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int bs = p.c.bs, Hkv = p.c.Hkv, G = p.c.G;
  const int bs_log2 = __builtin_ctz((unsigned)bs);
  const int T = p.split_tokens;
  auto n_tiles_of = [&](int qn) { return (qn * G + 15) / 16; };
  auto n_groups = [&](int qn) { return (n_tiles_of(qn) + RT - 1) / RT; };
  auto shared_seq = [&](int qn) { return kShared && n_tiles_of(qn) >= kShareMinTiles; };
  if constexpr (BAL) {
    attn_varlen_balanced<D, RT, FP8>(p, s_pb, s_pref, s_upref, s_wave, s_kv);
    return;
  }
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
    const int e0 = t0 >> bs_log2;
    const int n_ent = T >> bs_log2;
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
      const int ei = (tok >> bs_log2) - e0;        // bs is a power of two: no division
      const int xr = s_pb[ei < n_ent ? ei : 0];    // read unconditionally, in bounds
      const int x = ei < n_ent ? xr : -1;
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
        attend_shared<D, FP8>(p.c, g_sh, (span + 15) / 16, desc, t0, tiles, s_kv);
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
// Balanced schedule: a work unit (sequence, KV head on the shared path, group of row
// tiles) covers tiles [P, P + work) of the flattened space; workgroups w_a .. w_b
// held them and left partial rows in slots w + (global unit index). The units are
// taken grid-stride, each merging all of its rows.
template <int D>
__device__ __forceinline__ void attn_varlen_combine_balanced(const VarlenParams& p, int* s_pref,
                                                             int* s_upref, int* s_wave) {
  constexpr int TPR = D / 4;
  const int G = p.c.G, Hq = p.c.Hq, Hkv = p.c.Hkv;
  const bool share_ok = p.share_ok != 0;
  const long long W = sequence_prefix(p.B, s_pref, s_wave, [&](int b) {
    const SeqGeom sg = seq_geom(p, b, share_ok, p.rt);
    return sg.heads * head_tiles(sg, G);
  });
  const int U = sequence_prefix(p.B, s_upref, s_wave, [&](int b) {
    const SeqGeom sg = seq_geom(p, b, share_ok, p.rt);
    return sg.heads * sg.n_grp;
  });
  const long long N = p.nwg;
  const bool gaps = W < N;   // only then can a workgroup inside a unit's range hold no tile
  // One (work unit, 16-row block) per iteration; the unit's covering workgroups come
  // from the attention kernel, which recorded them at the unit's first tile.
  const long long items = (long long)U * p.slot_rows;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int k = (int)(it / p.slot_rows), rb = (int)(it - (long long)k * p.slot_rows);
    const int b = sequence_of(s_upref, p.B, k);
    const SeqGeom sg = seq_geom(p, b, share_ok, p.rt);
    const int local = k - s_upref[b];
    const int hu = local / sg.n_grp, grp = local - hu * sg.n_grp;
    const int n_heads = sg.shared ? 1 : Hkv;
    if (rb >= n_heads * sg.grp_rt) continue;
    const int t = rb % sg.grp_rt, hh = rb / sg.grp_rt;
    const int m0 = 16 * (grp * sg.grp_rt + t);
    const int rows = sg.qn * G;
    if (m0 >= rows) continue;
    const int n_rows = rows - m0 < 16 ? rows - m0 : 16;
    int w_a = 0, n_units = 0;
    if (group_tiles(sg, G, grp) > 0) {
      w_a = p.unit_info[2 * k];
      n_units = p.unit_info[2 * k + 1];
    }
    auto live = [&](int x) {
      if (!gaps) return true;
      const long long ww = w_a + x;
      return ww * W / N < (ww + 1) * W / N;
    };
    const int g = sg.shared ? hu : hh;
    const int srow = sg.shared ? t : hh * sg.grp_rt + t;
    const size_t blk0 = ((size_t)w_a + k) * p.slot_rows + srow;
    for (int i = threadIdx.x; i < n_rows * TPR; i += kCombineThreads) {
      const int rr = i / TPR, c4 = i - rr * TPR;
      const float* lse0 = p.part_lse + blk0 * 16 + rr;
      const float* o0 = p.part_o + (blk0 * 16 + rr) * D + 4 * c4;
      const f32x4 o = merge_rows<8>(n_units, lse0, (size_t)p.slot_rows * 16, o0,
                                    (size_t)p.slot_rows * 16 * D, live);
      const int m = m0 + rr, j = m / G;
      *(f32x4*)(p.out + ((size_t)(sg.q0 + j) * Hq + (size_t)g * G + (m - j * G)) * D + 4 * c4) = o;
    }
  }
  // Sequences with query rows but nothing to attend (empty context) have no unit:
  // their rows are zeros.
  for (int b = blockIdx.x; b < p.B; b += gridDim.x) {
    const SeqGeom sg = seq_geom(p, b, share_ok, p.rt);
    if (sg.n_grp > 0 || sg.qn <= 0) continue;
    for (int i = threadIdx.x; i < sg.qn * Hq * TPR; i += kCombineThreads)
      *(f32x4*)(p.out + (size_t)sg.q0 * Hq * D + 4 * (size_t)i) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

template <int D>
__global__ __launch_bounds__(kCombineThreads) void attn_varlen_combine_kernel(const VarlenParams p) {
  __shared__ int s_pref[kMaxBalBatch + 1];
  __shared__ int s_wave[kWaves];
  constexpr int TPR = D / 4;   // threads per row, 4 channels each
  const int G = p.c.G, Hq = p.c.Hq, Hkv = p.c.Hkv;
  if (p.balanced) {
    __shared__ int s_upref[kMaxBalBatch + 1];
    attn_varlen_combine_balanced<D>(p, s_pref, s_upref, s_wave);
    return;
  }
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
      const f32x4 o = merge_rows<8>(n_units, lse0, 16, o0, (size_t)16 * D, [](int) { return true; });
      const int m = m0 + rr, j = m / G;
      *(f32x4*)(p.out + ((size_t)(q0 + j) * Hq + (size_t)g * G + (m - j * G)) * D + 4 * c4) = o;
    }
  }
}

// Multi-token queries: row tiles per sequence, split size and workspace.
constexpr long long kVarlenMaxUnits = 1LL << 18;   // partial-row blocks (about 2 GB at D = 128)
constexpr int kVarlenRT = 2;   // row tiles per wave when a chunk spans more than one tile

struct VarlenPlan {
  int n_rt, split_tokens, num_splits;
  size_t o_bytes, lse_bytes;
  // Balanced schedule: workgroups, row tiles per partial slot, and its workspace.
  int rt, nwg, slot_rows, bal_grid;   // nwg shares over bal_grid workgroups
  size_t bal_o_bytes, bal_lse_bytes, bal_info_bytes;
  bool bal_ok;   // the flattened tile space fits the kernel's 32-bit prefix sums
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

  // Balanced schedule. Units: at most H_kv * (ceil(rt / 8) + 1) per sequence on the
  // shared path and ceil(rt / RT) + 1 on the per-head path, each covering at most
  // ceil(max_ctx / 32) tiles. Workgroups: all resident at once (two per CU with
  // row-tile pairs, three with single row tiles), and enough that no share holds
  // more tiles than one staged block-table chunk covers.
  pl.rt = pl.n_rt > 1 ? kVarlenRT : 1;
  pl.slot_rows = kShareTiles > pl.rt * Hkv ? kShareTiles : pl.rt * Hkv;
  const long long total_rt = ((long long)total_q * G + 15) / 16 + B;
  const long long u_bound = (long long)Hkv * ((total_rt + kShareTiles - 1) / kShareTiles + B) +
                            (total_rt + pl.rt - 1) / pl.rt + B;
  const long long w_bound = u_bound * (((long long)max_ctx + 31) / 32);
  pl.bal_ok = w_bound < (1LL << 31);
  const long long seg_cap = (long long)(kMaxTable - 1) * bs / 32 - 1;
  // The grid: two workgroups per CU with row-tile pairs (one wave's MFMA work hides
  // the other's loads); one with single row tiles, which stream K / V like decode
  // (58 single-token rows on 8K contexts: 162 us at one per CU, 175 at two, 192 at
  // three). Each workgroup takes the same number of consecutive shares, enough that
  // no share spans more tiles than one staged table chunk.
  const long long grid = (long long)(pl.rt == 1 ? 1 : 2) * balanced_capacity();
  const long long need = (w_bound + seg_cap - 2) / (seg_cap - 1);
  long long per = (need + grid - 1) / grid;
  if (per < 1) per = 1;
  if (grid * per > (1LL << 30)) per = (1LL << 30) / grid;
  pl.bal_grid = (int)grid;
  pl.nwg = (int)(grid * per);
  const size_t slots = (size_t)pl.nwg + (size_t)u_bound;
  pl.bal_o_bytes = align256(slots * pl.slot_rows * 16 * D * sizeof(float));
  pl.bal_lse_bytes = align256(slots * pl.slot_rows * 16 * sizeof(float));
  pl.bal_info_bytes = align256((size_t)u_bound * 2 * sizeof(int));
  return pl;
}

// The balanced schedule by default: on the 8K-average mixed batch (six chunks of
// 32-512 tokens, 58 single tokens) 464 us against 502 us with fixed 2048-position
// splits, and on eight 512-token chunks 984 against 1010 us (MI355X). Timestamps show
// every workgroup then holds 131-132 tiles and ends between 285 and 402 us: what
// remains is the per-tile cost, which varies with what shares the CU.
// GPKV_VARLEN_SCHEDULE=split|balanced forces the schedule (tuning and test switch,
// read per call); the workspace fits either wherever the balanced one can run.
static bool varlen_balanced() {
  const char* f = getenv("GPKV_VARLEN_SCHEDULE");
  if (f && strcmp(f, "split") == 0) return false;
  return true;
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
  const size_t split = pl.o_bytes + pl.lse_bytes,
               bal = pl.bal_ok ? pl.bal_o_bytes + pl.bal_lse_bytes + pl.bal_info_bytes : 0;
  return split > bal ? split : bal;
}

template <bool FP8, bool BAL>
static void launch_varlen_sched(bool multi, int head_dim, dim3 grid, dim3 block, hipStream_t s,
                                const VarlenParams& vp) {
  if (!multi) {
    if (head_dim == 128)
      attn_varlen_kernel<128, 1, FP8, BAL><<<grid, block, 0, s>>>(vp);
    else
      attn_varlen_kernel<64, 1, FP8, BAL><<<grid, block, 0, s>>>(vp);
  } else {
    if (head_dim == 128)
      attn_varlen_kernel<128, kVarlenRT, FP8, BAL><<<grid, block, 0, s>>>(vp);
    else
      attn_varlen_kernel<64, kVarlenRT, FP8, BAL><<<grid, block, 0, s>>>(vp);
  }
}

// One kernel instance per schedule: the schedule's outer loop is all that surrounds
// the tile loop in each (the tile loop runs at the register limit, so the outer
// code's live state shapes its code).
template <bool FP8>
static void launch_varlen(bool multi, int head_dim, dim3 grid, dim3 block, hipStream_t s,
                          const VarlenParams& vp) {
  if (vp.balanced)
    launch_varlen_sched<FP8, true>(multi, head_dim, grid, block, s, vp);
  else
    launch_varlen_sched<FP8, false>(multi, head_dim, grid, block, s, vp);
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
  // Batches whose (unit, tile) space would overflow the balanced kernel's 32-bit
  // prefix sums (very long contexts times long chunks) take the fixed splits.
  const bool balanced = varlen_balanced() && pl.bal_ok;
  const size_t need = balanced ? pl.bal_o_bytes + pl.bal_lse_bytes + pl.bal_info_bytes
                               : pl.o_bytes + pl.lse_bytes;
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
  vp.part_lse = (float*)((char*)workspace + (balanced ? pl.bal_o_bytes : pl.o_bytes));
  vp.unit_info = (int*)((char*)workspace + pl.bal_o_bytes + pl.bal_lse_bytes);   // balanced only
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
  vp.balanced = balanced ? 1 : 0;
  vp.slot_rows = pl.slot_rows;
  vp.nwg = pl.nwg;
  vp.rt = pl.rt;
  vp.share_ok = pl.rt > 1 ? 1 : 0;
  // One row tile per wave for decode-sized chunks; otherwise kVarlenRT tiles share
  // every K / V tile a wave loads. Both kernels take their work units grid-stride
  // from a fixed grid of at most four workgroups per CU.
  const int rt_per_wave = pl.n_rt > 1 ? kVarlenRT : 1;
  const long long tiles = ((long long)total_q * vp.c.G + 15) / 16 + batch;
  const long long units_max = (tiles / rt_per_wave + batch) * pl.num_splits;
  const long long cap = 4LL * balanced_capacity();
  const dim3 grid(balanced ? (unsigned)pl.bal_grid : (unsigned)(units_max < cap ? units_max : cap)),
      block(kWaves * 64);
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
