// Internal helpers shared by the host files of libpkv (not part of the ABI).
#pragma once

#include <cstdint>

#include "pkv.h"

namespace pkv {

// Record a thread-local error message and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the thread-local message (successful calls leave it untouched).
void clear_error();

// PKV_OK or INVALID_ARG/UNSUPPORTED with a message.
int validate_config(const pkv_config* cfg);

// Blocks of a pool (its configuration's num_blocks).
int32_t pool_num_blocks(const pkv_pool* pool);

inline int64_t elem_bytes(int32_t dtype) { return dtype == PKV_I8 ? 1 : 2; }

// Elements in one (layer, block, KV head) tile: 16 rows of D.
inline int64_t tile_elems(const pkv_config& c) { return int64_t(PKV_BLOCK_TOKENS) * c.head_dim; }
// Elements of one layer of the K (or V) region: N * Hkv tiles.
inline int64_t layer_elems(const pkv_config& c) {
  return int64_t(c.num_blocks) * c.num_kv_heads * tile_elems(c);
}
// Bytes of the whole K (or V) region.
inline int64_t region_bytes(const pkv_config& c) {
  return int64_t(c.num_layers) * layer_elems(c) * elem_bytes(c.dtype);
}

}  // namespace pkv
