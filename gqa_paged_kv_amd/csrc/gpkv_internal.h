// Internal helpers shared by the gpkv HIP translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gpkv.h"

namespace gpkv {

// ---------------------------------------------------------------------------
// Host side: status plumbing
// ---------------------------------------------------------------------------

// Records a formatted message for gpkv_last_error_message() and returns status.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the per-thread message (called on entry of every public function).
void clear_error();
// Maps hipGetLastError() after a launch to GPKV_OK / GPKV_ERR_HIP.
int check_launch(const char* what);
// Compute units of the current device (defined in paged_attention.hip): the
// balanced attention schedule runs one workgroup per CU.
int balanced_capacity();

inline bool supported_head_dim(int d) { return d == 64 || d == 128; }
inline bool supported_block_size(int bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }
constexpr int kMaxGroup = 16;

// Tokens per split-KV work unit (a multiple of 128); identical for the workspace
// query and the launch.
int split_tokens_for(int batch, int num_kv_heads, int span_tokens);
// The GPKV_SPLIT_TOKENS override (0 when unset or invalid).
int env_split_tokens();

// ---------------------------------------------------------------------------
// Device side
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer descriptor dword 3 for gfx9-family (CDNA) parts.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferFlags);
}

// Cache-policy bits of a buffer load on gfx950: NT (non-temporal) marks data that
// is streamed once. The KV cache is read exactly once per decode step, and NT loads
// sustain far more HBM bandwidth than default-policy loads on MI355X.
constexpr int kLoadNT = 2;

// Buffer loads: an offset at or past `bytes` of the descriptor returns zeros.
// AUX = kLoadNT streams data read once; AUX = 0 keeps it in the caches for
// readers that share it.
template <int AUX = kLoadNT>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}
template <int AUX = kLoadNT>
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX);
}
template <int AUX = kLoadNT>
__device__ __forceinline__ unsigned buf_load4(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX);
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Quest key min / max of a block after one more row k (eight bf16 channels per
// vector): the element-wise min and max of the block's current metadata and k,
// bf16 values compared as float (exact: each result is one of the inputs).
__device__ __forceinline__ void fold_min_max(const u32x4& k, const u32x4& om, const u32x4& ox,
                                             u32x4& mn, u32x4& mx) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float klo = bf16_lo(k[w]), khi = bf16_hi(k[w]);
    mn[w] = (__float_as_uint(fminf(bf16_lo(om[w]), klo)) >> 16) |
            (__float_as_uint(fminf(bf16_hi(om[w]), khi)) & 0xffff0000u);
    mx[w] = (__float_as_uint(fmaxf(bf16_lo(ox[w]), klo)) >> 16) |
            (__float_as_uint(fmaxf(bf16_hi(ox[w]), khi)) & 0xffff0000u);
  }
}

// v_perm_b32 helpers: pack the low (or high) 16-bit halves of a and b as (a | b << 16).
__device__ __forceinline__ unsigned pack_lo16(unsigned a, unsigned b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ unsigned pack_hi16(unsigned a, unsigned b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---------------------------------------------------------------------------
// FP8 (OCP E4M3: bias 7, no infinities, largest finite 448, NaN = S.1111.111)
// ---------------------------------------------------------------------------

// Nearest E4M3 code of a float32, ties to the even code, |y| > 448 saturating to
// 448, NaN -> 0x7F; the sign bit is y's. Integer arithmetic on the float32 bits.
__device__ __forceinline__ unsigned e4m3_from_f32(float y) {
  const unsigned u = __float_as_uint(y);
  const unsigned sign = (u >> 24) & 0x80u;
  const unsigned a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;             // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;     // |y| >= 448 (and inf)
  if (a < 0x3c800000u) {                         // |y| < 2^-6: steps of 2^-9
    const float t = __uint_as_float(a) * 512.0f;  // exact, t < 8
    return sign | (unsigned)__builtin_rintf(t);  // ties to even; 8 is the first normal
  }
  // Normal: keep 3 of the 23 mantissa bits, rounding to nearest even.
  const unsigned r = a + 0x7ffffu + ((a >> 20) & 1u);
  const unsigned code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
  return sign | code;                            // a < 448 keeps code <= 0x7e
}

// Four E4M3 codes (one per byte of w, lowest byte first) -> four bf16 values
// packed two per word. Every E4M3 value is exact in bf16; gfx950 converts a code
// pair straight to packed bf16 (scale 1: the same bits as decoding to float32 and
// keeping the high half, on all 256 codes), one instruction per two codes.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(unsigned w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);   // bytes 0, 1
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);    // bytes 2, 3
  return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Sixteen bf16 values (a: the first eight, b: the next eight) as OCP E4M3 codes of
// x * inv, one byte each in order (the FP8 write path's quantisation).
__device__ __forceinline__ u32x4 quantize16(u32x4 a, u32x4 b, float inv) {
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4& src = j < 2 ? a : b;
    const unsigned w0 = src[(2 * j) & 3], w1 = src[(2 * j + 1) & 3];
    const float y0 = bf16_lo(w0) * inv, y1 = bf16_hi(w0) * inv;
    const float y2 = bf16_lo(w1) * inv, y3 = bf16_hi(w1) * inv;
    out[j] = e4m3_from_f32(y0) | (e4m3_from_f32(y1) << 8) | (e4m3_from_f32(y2) << 16) |
             (e4m3_from_f32(y3) << 24);
  }
  return out;
}

// E4M3 codes are sign-magnitude, and among the finite codes of one sign a larger
// magnitude field is a larger magnitude. Flipping the sign bit of a non-negative
// code and every bit of a negative one gives bytes whose unsigned order is the
// order of the values (-448 -> 0x01 ... -0 -> 0x7F, +0 -> 0x80 ... 448 -> 0xFE;
// the two zeros stay distinct but adjacent). Four codes per word, one per byte.
__device__ __forceinline__ unsigned e4m3_order_bytes(unsigned w) {
  const unsigned neg = (w >> 7) & 0x01010101u;
  return w ^ (neg * 0x7Fu) ^ 0x80808080u;
}
__device__ __forceinline__ unsigned e4m3_from_order_bytes(unsigned k) {
  const unsigned t = k ^ 0x80808080u;
  return t ^ (((t >> 7) & 0x01010101u) * 0x7Fu);
}
// Per-byte unsigned min / max of two words.
__device__ __forceinline__ unsigned bytes_min(unsigned a, unsigned b) {
  unsigned r = 0;
#pragma unroll
  for (int i = 0; i < 32; i += 8) r |= min((a >> i) & 0xFFu, (b >> i) & 0xFFu) << i;
  return r;
}
__device__ __forceinline__ unsigned bytes_max(unsigned a, unsigned b) {
  unsigned r = 0;
#pragma unroll
  for (int i = 0; i < 32; i += 8) r |= max((a >> i) & 0xFFu, (b >> i) & 0xFFu) << i;
  return r;
}

// fold_min_max over sixteen E4M3 codes: the codes of the element-wise smaller and
// larger value of the block's current metadata (om, ox) and the new row k. Each
// result is one of the inputs (a zero extreme may come out as either zero code).
__device__ __forceinline__ void fold_min_max_e4m3(const u32x4& k, const u32x4& om,
                                                  const u32x4& ox, u32x4& mn, u32x4& mx) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const unsigned kk = e4m3_order_bytes(k[w]);
    mn[w] = e4m3_from_order_bytes(bytes_min(e4m3_order_bytes(om[w]), kk));
    mx[w] = e4m3_from_order_bytes(bytes_max(e4m3_order_bytes(ox[w]), kk));
  }
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Reductions over the four 16-lane rows of a wave (lanes r, r + 16, r + 32, r + 48
// all receive the result, bit-identical): gfx950's permlane swaps exchange rows
// 1 and 3 of one copy with rows 0 and 2 of another (16), and the upper half of one
// with the lower half of the other (32), in VALU with no LDS round trip.
__device__ __forceinline__ float max_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Cross-lane steps on DPP (a VALU operand modifier, a few cycles) rather than
// LDS permutes: row_shr:n moves lane i - n of the same 16-lane row into lane i,
// and a lane whose source falls outside its row reads 0 (bound_ctrl).
template <int N>
__device__ __forceinline__ unsigned row_shr_zero(unsigned v) {
  static_assert(N >= 1 && N <= 15, "row_shr takes 1..15");
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 + N, 0xF, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave (every lane active): a
// Hillis-Steele scan inside each 16-lane row, then the totals of the rows below
// (lanes 15, 31, 47) added from scalar registers.
__device__ __forceinline__ unsigned wave_inclusive_scan(unsigned v) {
  v += row_shr_zero<1>(v);
  v += row_shr_zero<2>(v);
  v += row_shr_zero<4>(v);
  v += row_shr_zero<8>(v);
  const unsigned r0 = (unsigned)__builtin_amdgcn_readlane((int)v, 15);
  const unsigned r1 = (unsigned)__builtin_amdgcn_readlane((int)v, 31);
  const unsigned r2 = (unsigned)__builtin_amdgcn_readlane((int)v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Bitwise OR over the 64 lanes of a wave (every lane active), the same in all lanes.
__device__ __forceinline__ unsigned wave_or(unsigned v) {
  v |= row_shr_zero<1>(v);
  v |= row_shr_zero<2>(v);
  v |= row_shr_zero<4>(v);
  v |= row_shr_zero<8>(v);   // lane 15 of each row now holds the row's OR
  return (unsigned)(__builtin_amdgcn_readlane((int)v, 15) | __builtin_amdgcn_readlane((int)v, 31) |
                    __builtin_amdgcn_readlane((int)v, 47) | __builtin_amdgcn_readlane((int)v, 63));
}

}  // namespace gpkv
