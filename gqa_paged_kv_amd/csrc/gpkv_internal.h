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

inline bool supported_head_dim(int d) { return d == 64 || d == 128; }
inline bool supported_block_size(int bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }
constexpr int kMaxGroup = 16;

// Tokens per split-KV work unit (a multiple of 128); identical for the workspace
// query and the launch.
int split_tokens_for(int batch, int num_kv_heads, int span_tokens);

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
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kLoadNT);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kLoadNT);
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// v_perm_b32 helpers: pack the low (or high) 16-bit halves of a and b as (a | b << 16).
__device__ __forceinline__ unsigned pack_lo16(unsigned a, unsigned b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ unsigned pack_hi16(unsigned a, unsigned b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace gpkv
