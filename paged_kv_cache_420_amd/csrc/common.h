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

}  // namespace pkv
