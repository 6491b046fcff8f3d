// Quest block scoring and Top-K selection, device side: shared by the selection
// kernels and by the one-launch Quest decode (selection, then attention over the
// selected blocks).
//
// ["Ascend Kernel-to-Serving Pipeline", section "Quest Sparse Attention"]: every
// logical block gets the classic Quest bound of q.k from its per-channel key
// minimum and maximum; the selection is per KV head, with the group's query heads
// summed. Because kmin <= kmax,
//   sum_h max(q_h*kmin, q_h*kmax) = kmax * sum_{q_h>0} q_h + kmin * sum_{q_h<0} q_h,
// so each (b, g) pre-reduces its queries once into two float64 vectors and a block
// costs 2*D float64 FMAs. Scores stay in float64; ties go to the lower logical block.
// Over E4M3 caches the metadata holds the codes of each channel's extremes and the
// bound is taken on the code values (the per-KV-head key scale, one positive factor
// for every block of a head, leaves the selection unchanged): the same kernels with
// FP8 = true read 8 bytes of codes where they read 16 bytes of bf16.
#pragma once

#include <math.h>

#include "gpkv_internal.h"

namespace gpkv {

// Metadata loads of the score kernels: each row is read once per step, and
// non-temporal loads measured faster than default-policy ones here too.
__device__ __forceinline__ u32x4 meta_load(const u32x4* ptr) { return __builtin_nontemporal_load(ptr); }

// Eight channels of a metadata row starting at element `elem` (a multiple of 8):
// 16 bytes of bf16, or 8 bytes of E4M3 codes in words 0 and 1.
template <bool FP8>
__device__ __forceinline__ u32x4 meta_load8(const void* base, size_t elem) {
  if constexpr (FP8) {
    const u32x2 x = __builtin_nontemporal_load((const u32x2*)((const unsigned char*)base + elem));
    return u32x4{x[0], x[1], 0u, 0u};
  } else {
    return meta_load((const u32x4*)((const unsigned short*)base + elem));
  }
}

// A block's bound over the lane's D / 8 channels (64v + 8 sub .. + 8 for v < D / 64):
// kmax against the positive query sums, kmin against the negative ones.
template <int D, bool FP8>
__device__ __forceinline__ double bound_lane(const u32x4 (&mn)[D / 64], const u32x4 (&mx)[D / 64],
                                             const double* s_pos, const double* s_neg, int sub) {
  double acc = 0.0;
#pragma unroll
  for (int v = 0; v < D / 64; ++v) {
    if constexpr (FP8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {   // word h: channels 4h .. 4h + 3, as bf16 pairs
        const u32x2 lo = e4m3x4_to_bf16(mn[v][h]), hi = e4m3x4_to_bf16(mx[v][h]);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int j = (v * 8 + 4 * h + 2 * k) * 8 + sub;   // qb_index of channel 64v + 8 sub + 4h + 2k
          acc = fma((double)bf16_lo(hi[k]), s_pos[j], acc);
          acc = fma((double)bf16_lo(lo[k]), s_neg[j], acc);
          acc = fma((double)bf16_hi(hi[k]), s_pos[j + 8], acc);
          acc = fma((double)bf16_hi(lo[k]), s_neg[j + 8], acc);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = (v * 8 + 2 * k) * 8 + sub;   // qb_index of channel 64v + 8 sub + 2k
        acc = fma((double)bf16_lo(mx[v][k]), s_pos[j], acc);
        acc = fma((double)bf16_lo(mn[v][k]), s_neg[j], acc);
        acc = fma((double)bf16_hi(mx[v][k]), s_pos[j + 8], acc);
        acc = fma((double)bf16_hi(mn[v][k]), s_neg[j + 8], acc);
      }
    }
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Scores: one float64 per (sequence, KV head, logical block)
// ---------------------------------------------------------------------------

constexpr int kSelectThreads = 256;       // two-kernel path
constexpr int kMaxSelectThreads = 1024;   // fused path: up to 128 blocks per pass
constexpr int kScoreUnroll = 4;           // passes of loads in flight (two-kernel path)
constexpr int kFusedUnroll = 4;           // ... (fused path: block-table row staged in LDS)
constexpr int kFusedThreads = 512;        // fused path: 2 waves per SIMD (no spills at 4 passes)
constexpr int kScoreBlocksPerWG = kSelectThreads / 8 * kScoreUnroll;   // two-kernel path
constexpr int kMaxLdsKeys = 6144;        // keys of one (b, g) that fit in LDS (48 KB)
constexpr int kMaxFusedBlocks = 4096;    // fused path: keys + block-table row (48 KB)

struct ScoreParams {
  double* scores;              // [B, H_kv, max_blocks] (two-kernel path)
  int* out;                    // [B, H_kv, K] (fused path)
  const unsigned short* q;     // [B, H_q, D]
  const void* kmin;            // [NB, H_kv, D] bf16, or E4M3 codes (the FP8 kernels)
  const void* kmax;
  const int* bt;
  const int* ctx;
  long long NB;
  int Hq, Hkv, G, bs, max_blocks, max_ctx, K;
};

__device__ __forceinline__ unsigned long long score_key(double x) {
  if (x == 0.0) x = 0.0;  // +0 and -0 are equal scores: give them one key
  const long long bits = __double_as_longlong(x);
  return bits < 0 ? ~(unsigned long long)bits : ((unsigned long long)bits | 0x8000000000000000ull);
}

// Channels of a score lane: the eight lanes (sub = 0..7) of a block read its
// metadata row in 128-byte pieces, lane sub taking channels 64v + 8 sub .. +8 for
// v < D/64, so each load instruction covers whole 128-byte lines. The per-channel
// query sums sit in LDS at ((c / 64) * 8 + c % 8) * 8 + (c / 8) % 8: for a given
// (v, channel pair) the eight lanes of a block read eight consecutive doubles (no
// bank conflicts). Per KV head the arrays are padded to D + 8.
template <int D>
__device__ __forceinline__ int qb_index(int c) {
  return ((c >> 6) * 8 + (c & 7)) * 8 + ((c >> 3) & 7);
}
constexpr int kQbPad = 8;

// Query rows of heads [h0, h0 + nh) of sequence b into LDS as raw bf16, with one
// round of 16-byte loads (nh * D * 2 bytes).
template <int D>
__device__ __forceinline__ void stage_query(const ScoreParams& p, int b, int h0, int nh,
                                            unsigned short* s_q) {
  const u32x4* src = (const u32x4*)(p.q + ((size_t)b * p.Hq + h0) * D);
  u32x4* dst = (u32x4*)s_q;
  for (int i = threadIdx.x; i < nh * D / 8; i += blockDim.x) dst[i] = src[i];
}

// pos[c] = sum of the positive q[h][c] over the G heads of a group, neg[c] = sum of
// the negative ones, in head order (the exact identity of the block bound needs
// only kmin <= kmax). s_qg holds the group's G query rows.
template <int D>
__device__ __forceinline__ void group_bounds(const unsigned short* s_qg, int G, int c,
                                             double* pos_out, double* neg_out) {
  double pos = 0.0, neg = 0.0;
  for (int h = 0; h < G; ++h) {
    const double v = (double)__uint_as_float((unsigned)s_qg[h * D + c] << 16);
    if (v > 0.0)
      pos += v;
    else
      neg += v;
  }
  *pos_out = pos;
  *neg_out = neg;
}

// s_pos / s_neg for one (b, g); s_q is scratch LDS for G * D bf16. Ends with a
// barrier.
template <int D>
__device__ __forceinline__ void query_bounds(const ScoreParams& p, int b, int g, unsigned short* s_q,
                                             double* s_pos, double* s_neg) {
  stage_query<D>(p, b, g * p.G, p.G, s_q);
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += blockDim.x)
    group_bounds<D>(s_q, p.G, c, s_pos + qb_index<D>(c), s_neg + qb_index<D>(c));
  __syncthreads();
}

// Scores of logical blocks lb0 + P*u + slot (P = blockDim/8 blocks per pass,
// u < UNROLL) for one (b, g): eight lanes per block (sub = lane & 7) each
// take D/8 channels, all loads are issued before any arithmetic, and xor shuffles
// merge the eight partial sums. pb_at(lb) gives the physical block of lb < nb (any
// value outside [0, NB) scores as -inf). Calls emit(lb, key) from the sub == 0 lane
// of every block lb < nb. Every lane of the workgroup must call this with the same
// lb0. FP8: the metadata holds E4M3 codes and the bound is taken on their values.
template <int D, bool FP8, int UNROLL, class PbAt, class Emit>
__device__ __forceinline__ void score_blocks(const ScoreParams& p, int g, int nb, int lb0,
                                             const PbAt& pb_at, const double* s_pos,
                                             const double* s_neg, const Emit& emit) {
  constexpr int NV = D / 64;      // 16-byte vectors per lane per array
  const int sub = threadIdx.x & 7, slot = threadIdx.x >> 3;
  const int P = blockDim.x >> 3;
  u32x4 mn[UNROLL][NV], mx[UNROLL][NV];
  bool ok[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int lb = lb0 + P * u + slot;
    const int pb = lb < nb ? pb_at(lb) : -1;
    ok[u] = pb >= 0 && pb < p.NB;
    const size_t o = ((size_t)(ok[u] ? pb : 0) * p.Hkv + g) * D + (size_t)sub * 8;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      mn[u][v] = ok[u] ? meta_load8<FP8>(p.kmin, o + 64 * v) : u32x4{0, 0, 0, 0};
      mx[u][v] = ok[u] ? meta_load8<FP8>(p.kmax, o + 64 * v) : u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    double acc = bound_lane<D, FP8>(mn[u], mx[u], s_pos, s_neg, sub);
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    const int lb = lb0 + P * u + slot;
    if (lb < nb && sub == 0) emit(lb, score_key(ok[u] ? acc : -INFINITY));
  }
}

// ---------------------------------------------------------------------------
// Top-K: radix select on order-preserving 64-bit keys, ties to the lower index
// ---------------------------------------------------------------------------

// Exclusive prefix sum of v over the workgroup's threads; *total receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = (int)wave_inclusive_scan((unsigned)v);
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    const int x = s_wave[w];
    off += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// Histogram and pass result are double-buffered: pass i uses buffer i & 1 and
// clears the other one for pass i + 1, so a pass needs two barriers (histogram
// complete; bucket found) and no barrier to clear or to retire what it read.
struct SelectShared {
  unsigned hist[2][256];
  int wave_sums[kMaxSelectThreads / 64];
  unsigned long long red_or[kMaxSelectThreads / 64];
  int digit[2], above[2], cnt[2];
};

// Writes the ascending ids of the K largest keys among key_at(0..n-1) (K < n) to
// out[0..K); equal keys are taken lowest index first. Keys are read through
// key_at; every thread of the workgroup must call this.
template <class KeyAt>
__device__ void radix_topk(int n, int K, const KeyAt& key_at, int* out, SelectShared& sh) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int C = (n + nt - 1) / nt;
  const int i0 = min(n, tid * C), i1 = min(n, i0 + C);
  for (int d = tid; d < 2 * 256; d += nt) (&sh.hist[0][0])[d] = 0;
  if (tid < 2) {
    sh.digit[tid] = 0;
    sh.above[tid] = 0;
    sh.cnt[tid] = 0;
  }
  // Bits every key shares need no pass: start at the highest bit where some key
  // differs from key 0 (so where keys differ at all).
  const unsigned long long k_ref = key_at(0);
  unsigned long long k_diff = 0ull;
  for (int i = i0; i < i1; ++i) k_diff |= key_at(i) ^ k_ref;
  k_diff = ((unsigned long long)wave_or((unsigned)(k_diff >> 32)) << 32) | wave_or((unsigned)k_diff);
  if ((tid & 63) == 0) sh.red_or[tid >> 6] = k_diff;
  __syncthreads();
  unsigned long long diff = 0ull;
  for (int w = 0; w < (nt >> 6); ++w) diff |= sh.red_or[w];
  const int top = diff ? 63 - __clzll((long long)diff) : -1;   // highest differing bit
  unsigned long long mask = top >= 63 ? 0ull : (~0ull << (top + 1));
  unsigned long long prefix = k_ref & mask;
  int need = K, shift = 0;
  bool whole = false;   // the last bucket is taken entirely (no tie to break)
  for (int pass = 0; top >= 0 && pass < 8; ++pass) {
    const int buf = pass & 1;
    shift = top - 7 - 8 * pass;
    if (shift < 0) shift = 0;
    // hist[buf] was cleared before the previous pass's first barrier (or before
    // the reduction's barrier above); hist[buf ^ 1] was last read by the previous
    // pass's bucket search, which every thread has passed.
    for (int i = i0; i < i1; ++i) {
      const unsigned long long key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[buf][(key >> shift) & 255], 1u);
    }
    for (int d = tid; d < 256; d += nt) sh.hist[buf ^ 1][d] = 0;
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending order of keys)
      unsigned c[4], t = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c[k] = sh.hist[buf][255 - 4 * tid - k];
        t += c[k];
      }
      const unsigned inc = wave_inclusive_scan(t);
      const unsigned excl = inc - t;
      if (excl < (unsigned)need && (unsigned)need <= inc) {
        unsigned above = excl;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (above + c[k] >= (unsigned)need) {
            sh.digit[buf] = 255 - 4 * tid - k;
            sh.above[buf] = (int)above;
            sh.cnt[buf] = (int)c[k];
            break;
          }
          above += c[k];
        }
      }
    }
    __syncthreads();
    // The next write of this buffer's result is two passes on, after a barrier
    // that every thread reaches only once it has read these.
    const int digit = sh.digit[buf], above = sh.above[buf], cnt = sh.cnt[buf];
    need -= above;
    prefix |= (unsigned long long)digit << shift;
    mask |= 0xFFull << shift;
    whole = cnt == need;
    if (whole || shift == 0) break;  // bucket fully selected, or every bit resolved
  }

  // Selected: keys above the resolved prefix, plus the first `need` (by index)
  // of those equal to it (all of them when the bucket is taken whole: then no
  // rank among equal keys is needed, and one scan is saved).
  const unsigned long long ref = prefix >> shift;
  int n_eq = 0, rank = 0, tot;
  if (whole) {
    need = n;
  } else {
    for (int i = i0; i < i1; ++i) n_eq += (key_at(i) >> shift) == ref;
    rank = block_exclusive_scan(n_eq, sh.wave_sums, &tot);
  }
  int n_sel = 0;
  for (int i = i0; i < i1; ++i) {
    const unsigned long long k = key_at(i) >> shift;
    if (k > ref) {
      ++n_sel;
    } else if (k == ref) {
      n_sel += rank < need;
      ++rank;
    }
  }
  int pos = block_exclusive_scan(n_sel, sh.wave_sums, &tot);
  rank -= n_eq;
  for (int i = i0; i < i1; ++i) {
    const unsigned long long k = key_at(i) >> shift;
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

__device__ __forceinline__ bool select_all(int n, int K, int* out) {
  if (K < n) return false;
  for (int i = threadIdx.x; i < K; i += blockDim.x) out[i] = i < n ? i : -1;
  return true;
}

}  // namespace gpkv
