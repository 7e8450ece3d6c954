// Shared internals of libpkv: status codes, error text, argument checks.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Records a printf-style message as the calling thread's last error and
// returns `code`, so call sites can write `return fail(PKV_ERR_INVALID, ...)`.
int32_t fail(int32_t code, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

// Clears the calling thread's last error and returns PKV_OK.
int32_t ok();

inline int dtype_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Prefix groups of one shared-prefix decode call: the batch's rows
// [start[g], start[g + 1]) were forked from one parent and share its first
// prefix_len[g] tokens (0: the group shares nothing).
constexpr int kMaxPrefixGroups = 128;
struct PrefixGroups {
  int32_t count;
  int32_t start[kMaxPrefixGroups + 1];
  int32_t prefix_len[kMaxPrefixGroups];
};

// prefill.hip: the prefix partials of the shared-prefix decode (arguments
// checked by the caller; returns the launch's hipError_t).  Every group's
// prefix is split into key ranges of split_keys keys; range z of group g
// goes to partial slot z of each of its rows.  The launch also writes each
// row's record row_info[4 r .. 4 r + 3] = {prefix_len, first row of its
// group, prefix slots, 0} for the suffix and merge launches.
int launch_prefix_partials(int32_t dtype, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           const PrefixGroups& groups, int32_t num_heads, int32_t num_kv_heads,
                           int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                           int32_t split_keys, int32_t max_splits, float scale, float* ws_acc,
                           float* ws_ml, int32_t* row_info, int32_t slots, void* stream);

// Rows per workgroup of the prefill kernel (the shared-prefix split count
// is chosen from the grid it gives).
constexpr int kPrefillRowsPerGroup = 256;

}  // namespace pkv
