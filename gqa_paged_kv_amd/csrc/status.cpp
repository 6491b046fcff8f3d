// Status strings, the per-thread error message and the split-size policy.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include "gpkv_internal.h"

namespace gpkv {

// Waves the split heuristic aims for (several times what the GPU holds at once).
constexpr long long kSplitTargetWaves = 8192;

static thread_local char g_msg[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_msg[0] = '\0'; }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GPKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return GPKV_OK;
}

// Split-KV sizing ([TL18] 4.1 and 8(5): too few splits starve the GPU, too many
// make the partial outputs and the extra combine launch dominate). A workgroup
// owns one (sequence, split) with one wave per KV head (at most 8), and MI355X
// keeps about 2048 such waves resident (256 CUs x 2 per SIMD at this kernel's
// register use). Take the longest split that still yields a few times that many
// waves, so each split's partial output stays a small fraction of the KV bytes it
// reads. The grid may only depend on host scalars, so the estimate uses the span
// (max_context_len, or topk_blocks * block_size for the sparse path).
// GPKV_SPLIT_TOKENS (a multiple of 128 in [128, 2048]) overrides the choice; it is
// read on every call so the workspace query and the launch always agree.
int env_split_tokens() {
  const char* s = getenv("GPKV_SPLIT_TOKENS");
  if (!s) return 0;
  const int x = atoi(s);
  if (x < 128 || x > 2048 || (x % 128) != 0) return 0;
  return x;
}

int split_tokens_for(int batch, int num_kv_heads, int span_tokens) {
  int forced = env_split_tokens();
  if (forced) return forced;
  const long long waves = (long long)batch * (num_kv_heads < 8 ? num_kv_heads : 8);
  int t = 2048;
  while (t > 128 && waves * ((span_tokens + t - 1) / t) < kSplitTargetWaves) t >>= 1;
  return t;
}

}  // namespace gpkv

extern "C" const char* gpkv_status_string(int status) {
  switch (status) {
    case GPKV_OK: return "ok";
    case GPKV_ERR_NULL: return "null pointer argument";
    case GPKV_ERR_SHAPE: return "invalid or inconsistent sizes";
    case GPKV_ERR_UNSUPPORTED: return "unsupported head_dim, block_size or group size";
    case GPKV_ERR_WORKSPACE: return "workspace missing or too small";
    case GPKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" const char* gpkv_last_error_message(void) { return gpkv::g_msg; }

extern "C" int32_t gpkv_split_tokens(int32_t batch, int32_t num_kv_heads, int32_t span_tokens) {
  return gpkv::split_tokens_for(batch, num_kv_heads, span_tokens);
}
