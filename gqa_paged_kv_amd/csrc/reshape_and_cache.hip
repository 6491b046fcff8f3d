// ReshapeAndCache: scatter new tokens' K/V rows into the paged cache.
//
// ["Ascend Kernel-to-Serving Pipeline", section "ReshapeAndCache"]: the physical
// block of a token is slot // block_size and its row inside the block is
// slot % block_size; a negative slot means the token is not written.
//
// With the cache laid out [num_blocks, block_size, H_kv, D], one token's K (or V)
// for all KV heads is a single contiguous row of H_kv * D bf16, so the write is a
// 16-byte-per-lane row copy. One wave per token: T is small (one new token per
// sequence), so the kernel is launch-bound and its only job is to move whole
// rows with full-width stores.
#include "gpkv_internal.h"

namespace gpkv {

__global__ __launch_bounds__(64) void reshape_and_cache_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value, u32x4* __restrict__ key_cache,
    u32x4* __restrict__ value_cache, const int64_t* __restrict__ slot_mapping, int row_vec,
    int block_size, long long num_slots) {
  const int i = blockIdx.x;
  const long long s = slot_mapping[i];
  if (s < 0 || s >= num_slots) return;  // negative: skip; past the pool: tolerated, skipped
  const long long blk = s / block_size;
  const long long off = s - blk * block_size;
  const size_t dst = (size_t)(blk * block_size + off) * (size_t)row_vec;
  const size_t src = (size_t)i * (size_t)row_vec;
  for (int c = threadIdx.x; c < row_vec; c += 64) {
    key_cache[dst + c] = key[src + c];
    value_cache[dst + c] = value[src + c];
  }
}


// Fused write path: the same row copy, plus an incremental update of the Quest
// key min / max of the block each token lands in (the token is the newest row of
// its block: row 0 starts the block's metadata afresh, any later row folds into
// the block's current metadata with min / max). Results are input values, so the
// update is exact.
__global__ __launch_bounds__(64) void reshape_and_cache_quest_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value, u32x4* __restrict__ key_cache,
    u32x4* __restrict__ value_cache, u32x4* __restrict__ key_min, u32x4* __restrict__ key_max,
    const int64_t* __restrict__ slot_mapping, int row_vec, int block_size, long long num_slots) {
  const int i = blockIdx.x;
  const long long s = slot_mapping[i];
  if (s < 0 || s >= num_slots) return;
  const long long blk = s / block_size;
  const long long off = s - blk * block_size;
  const size_t dst = (size_t)(blk * block_size + off) * (size_t)row_vec;
  const size_t src = (size_t)i * (size_t)row_vec;
  const size_t meta = (size_t)blk * (size_t)row_vec;
  for (int c = threadIdx.x; c < row_vec; c += 64) {
    const u32x4 k = key[src + c];
    key_cache[dst + c] = k;
    value_cache[dst + c] = value[src + c];
    u32x4 mn = k, mx = k;
    if (off > 0) fold_min_max(k, key_min[meta + c], key_max[meta + c], mn, mx);
    key_min[meta + c] = mn;
    key_max[meta + c] = mx;
  }
}


// FP8 write path: the same slot rule; each row is quantised to OCP E4M3 with its
// KV head's scale (quantize16: code = e4m3(x * (1 / scale)), both float32 operations,
// the reciprocal a correctly rounded division). 16 bf16 in, 16 bytes out per lane.
__global__ __launch_bounds__(64) void reshape_and_cache_fp8_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value, u32x4* __restrict__ key_cache,
    u32x4* __restrict__ value_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int64_t* __restrict__ slot_mapping, int row_vec8,
    int head_dim, int block_size, long long num_slots) {
  const int i = blockIdx.x;
  const long long s = slot_mapping[i];
  if (s < 0 || s >= num_slots) return;
  const int row_vec = row_vec8 / 2;   // 16-byte vectors of one E4M3 row
  const size_t dst = (size_t)s * (size_t)row_vec;
  const size_t src = (size_t)i * (size_t)row_vec8;
  for (int c = threadIdx.x; c < row_vec; c += 64) {
    const int g = (16 * c) / head_dim;
    const float kinv = 1.0f / k_scale[g], vinv = 1.0f / v_scale[g];
    key_cache[dst + c] = quantize16(key[src + 2 * c], key[src + 2 * c + 1], kinv);
    value_cache[dst + c] = quantize16(value[src + 2 * c], value[src + 2 * c + 1], vinv);
  }
}

// FP8 write path with the Quest fold: each row is quantised as above and its codes
// fold into the block's E4M3 key min / max (fold_min_max_e4m3: row 0 starts the
// block's metadata afresh, a later row takes the min / max of values).
__global__ __launch_bounds__(64) void reshape_and_cache_fp8_quest_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value, u32x4* __restrict__ key_cache,
    u32x4* __restrict__ value_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, u32x4* __restrict__ key_min, u32x4* __restrict__ key_max,
    const int64_t* __restrict__ slot_mapping, int row_vec8, int head_dim, int block_size,
    long long num_slots) {
  const int i = blockIdx.x;
  const long long s = slot_mapping[i];
  if (s < 0 || s >= num_slots) return;
  const long long blk = s / block_size;
  const long long off = s - blk * block_size;
  const int row_vec = row_vec8 / 2;
  const size_t dst = (size_t)s * (size_t)row_vec;
  const size_t src = (size_t)i * (size_t)row_vec8;
  const size_t meta = (size_t)blk * (size_t)row_vec;
  for (int c = threadIdx.x; c < row_vec; c += 64) {
    const int g = (16 * c) / head_dim;
    const float kinv = 1.0f / k_scale[g], vinv = 1.0f / v_scale[g];
    const u32x4 k = quantize16(key[src + 2 * c], key[src + 2 * c + 1], kinv);
    key_cache[dst + c] = k;
    value_cache[dst + c] = quantize16(value[src + 2 * c], value[src + 2 * c + 1], vinv);
    u32x4 mn = k, mx = k;
    if (off > 0) fold_min_max_e4m3(k, key_min[meta + c], key_max[meta + c], mn, mx);
    key_min[meta + c] = mn;
    key_max[meta + c] = mx;
  }
}

}  // namespace gpkv

extern "C" int gpkv_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                      void* value_cache, const int64_t* slot_mapping,
                                      int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int64_t num_blocks, void* stream) {
  using namespace gpkv;
  clear_error();
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0)
    return fail(GPKV_ERR_SHAPE, "reshape_and_cache: num_tokens=%d num_kv_heads=%d num_blocks=%lld",
                num_tokens, num_kv_heads, (long long)num_blocks);
  if (!supported_head_dim(head_dim))
    return fail(GPKV_ERR_UNSUPPORTED, "reshape_and_cache: head_dim=%d (64 or 128)", head_dim);
  if (!supported_block_size(block_size))
    return fail(GPKV_ERR_UNSUPPORTED, "reshape_and_cache: block_size=%d (16/32/64/128)", block_size);
  if (num_tokens == 0) return GPKV_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(GPKV_ERR_NULL, "reshape_and_cache: null pointer argument");
  const int row_vec = num_kv_heads * head_dim * 2 / 16;
  reshape_and_cache_kernel<<<dim3(num_tokens), dim3(64), 0, (hipStream_t)stream>>>(
      (const u32x4*)key, (const u32x4*)value, (u32x4*)key_cache, (u32x4*)value_cache,
      slot_mapping, row_vec, block_size, (long long)num_blocks * block_size);
  return check_launch("reshape_and_cache");
}

extern "C" int gpkv_reshape_and_cache_quest(const void* key, const void* value, void* key_cache,
                                            void* value_cache, void* key_min, void* key_max,
                                            const int64_t* slot_mapping, int32_t num_tokens,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int64_t num_blocks, void* stream) {
  using namespace gpkv;
  clear_error();
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0)
    return fail(GPKV_ERR_SHAPE,
                "reshape_and_cache_quest: num_tokens=%d num_kv_heads=%d num_blocks=%lld",
                num_tokens, num_kv_heads, (long long)num_blocks);
  if (!supported_head_dim(head_dim))
    return fail(GPKV_ERR_UNSUPPORTED, "reshape_and_cache_quest: head_dim=%d (64 or 128)", head_dim);
  if (!supported_block_size(block_size))
    return fail(GPKV_ERR_UNSUPPORTED, "reshape_and_cache_quest: block_size=%d (16/32/64/128)",
                block_size);
  if (num_tokens == 0) return GPKV_OK;
  if (!key || !value || !key_cache || !value_cache || !key_min || !key_max || !slot_mapping)
    return fail(GPKV_ERR_NULL, "reshape_and_cache_quest: null pointer argument");
  const int row_vec = num_kv_heads * head_dim * 2 / 16;
  reshape_and_cache_quest_kernel<<<dim3(num_tokens), dim3(64), 0, (hipStream_t)stream>>>(
      (const u32x4*)key, (const u32x4*)value, (u32x4*)key_cache, (u32x4*)value_cache,
      (u32x4*)key_min, (u32x4*)key_max, slot_mapping, row_vec, block_size,
      (long long)num_blocks * block_size);
  return check_launch("reshape_and_cache_quest");
}

extern "C" int gpkv_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                                          void* value_cache, const float* k_scale,
                                          const float* v_scale, const int64_t* slot_mapping,
                                          int32_t num_tokens, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          int64_t num_blocks, void* stream) {
  using namespace gpkv;
  clear_error();
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0)
    return fail(GPKV_ERR_SHAPE,
                "reshape_and_cache_fp8: num_tokens=%d num_kv_heads=%d num_blocks=%lld",
                num_tokens, num_kv_heads, (long long)num_blocks);
  if (!supported_head_dim(head_dim))
    return fail(GPKV_ERR_UNSUPPORTED, "reshape_and_cache_fp8: head_dim=%d (64 or 128)", head_dim);
  if (!supported_block_size(block_size))
    return fail(GPKV_ERR_UNSUPPORTED, "reshape_and_cache_fp8: block_size=%d (16/32/64/128)",
                block_size);
  if (num_tokens == 0) return GPKV_OK;
  if (!key || !value || !key_cache || !value_cache || !k_scale || !v_scale || !slot_mapping)
    return fail(GPKV_ERR_NULL, "reshape_and_cache_fp8: null pointer argument");
  const int row_vec8 = num_kv_heads * head_dim / 8;   // 16-byte vectors of one bf16 row
  reshape_and_cache_fp8_kernel<<<dim3(num_tokens), dim3(64), 0, (hipStream_t)stream>>>(
      (const u32x4*)key, (const u32x4*)value, (u32x4*)key_cache, (u32x4*)value_cache, k_scale,
      v_scale, slot_mapping, row_vec8, head_dim, block_size, (long long)num_blocks * block_size);
  return check_launch("reshape_and_cache_fp8");
}

extern "C" int gpkv_reshape_and_cache_fp8_quest(const void* key, const void* value,
                                                void* key_cache, void* value_cache,
                                                const float* k_scale, const float* v_scale,
                                                void* key_min, void* key_max,
                                                const int64_t* slot_mapping, int32_t num_tokens,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int64_t num_blocks,
                                                void* stream) {
  using namespace gpkv;
  clear_error();
  const char* fn = "reshape_and_cache_fp8_quest";
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0)
    return fail(GPKV_ERR_SHAPE, "%s: num_tokens=%d num_kv_heads=%d num_blocks=%lld", fn,
                num_tokens, num_kv_heads, (long long)num_blocks);
  if (!supported_head_dim(head_dim))
    return fail(GPKV_ERR_UNSUPPORTED, "%s: head_dim=%d (64 or 128)", fn, head_dim);
  if (!supported_block_size(block_size))
    return fail(GPKV_ERR_UNSUPPORTED, "%s: block_size=%d (16/32/64/128)", fn, block_size);
  if (num_tokens == 0) return GPKV_OK;
  if (!key || !value || !key_cache || !value_cache || !k_scale || !v_scale || !key_min ||
      !key_max || !slot_mapping)
    return fail(GPKV_ERR_NULL, "%s: null pointer argument", fn);
  const int row_vec8 = num_kv_heads * head_dim / 8;
  reshape_and_cache_fp8_quest_kernel<<<dim3(num_tokens), dim3(64), 0, (hipStream_t)stream>>>(
      (const u32x4*)key, (const u32x4*)value, (u32x4*)key_cache, (u32x4*)value_cache, k_scale,
      v_scale, (u32x4*)key_min, (u32x4*)key_max, slot_mapping, row_vec8, head_dim, block_size,
      (long long)num_blocks * block_size);
  return check_launch(fn);
}
