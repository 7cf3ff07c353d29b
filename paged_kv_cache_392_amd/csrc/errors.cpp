// Status strings, the thread-local last-error message and config validation.
#include <cstdarg>
#include <cstdio>

#include "pkv_internal.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace pkv {

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_last_error[0] = '\0'; }

int validate_config(const pkv_config* cfg) {
  if (!cfg) return fail(PKV_ERR_INVALID_ARG, "config is NULL");
  if (cfg->block_size != PKV_BLOCK_TOKENS)
    return fail(PKV_ERR_INVALID_ARG, "block_size must be 16 (got %d)", cfg->block_size);
  if (cfg->num_layers < 1 || cfg->num_blocks < 1 || cfg->num_kv_heads < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_layers, num_blocks and num_kv_heads must be >= 1");
  // slots are int32: block * 16 + offset must not overflow
  if (cfg->num_blocks > INT32_MAX / PKV_BLOCK_TOKENS)
    return fail(PKV_ERR_INVALID_ARG, "num_blocks too large for int32 slots");
  if (cfg->head_dim != 64 && cfg->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", cfg->head_dim);
  if (cfg->dtype != PKV_F16 && cfg->dtype != PKV_I8)
    return fail(PKV_ERR_UNSUPPORTED, "dtype %d not supported", cfg->dtype);
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

const char* pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_NO_BLOCKS: return "no free blocks";
    case PKV_ERR_UNKNOWN_SEQ: return "unknown sequence";
    case PKV_ERR_REFCOUNT: return "refcount inconsistency";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* pkv_last_error(void) { return g_last_error; }

int64_t pkv_pool_bytes(const pkv_config* cfg) {
  int st = pkv::validate_config(cfg);
  if (st != PKV_OK) return st;
  // 2 regions * L * N * Hkv * 16 * D * E, checked for int64 overflow
  int64_t bytes = 2 * PKV_BLOCK_TOKENS;
  const int64_t factors[] = {cfg->num_layers, cfg->num_blocks, cfg->num_kv_heads, cfg->head_dim,
                             pkv::elem_bytes(cfg->dtype)};
  for (int64_t f : factors)
    if (__builtin_mul_overflow(bytes, f, &bytes))
      return pkv::fail(PKV_ERR_INVALID_ARG, "pool size overflows int64");
  if (cfg->dtype == PKV_I8) {
    // one fp16 K scale and one V scale per (layer, block, KV head)
    int64_t scales = int64_t(cfg->num_layers) * cfg->num_blocks * cfg->num_kv_heads * 2 * 2;
    if (__builtin_add_overflow(bytes, scales, &bytes))
      return pkv::fail(PKV_ERR_INVALID_ARG, "pool size overflows int64");
  }
  return bytes;
}

}  // extern "C"
