// E4M3 encoding of 16-element row pieces, shared by every kernel that
// stores 8-bit cache codes (the slot-mapped append and the decode step's
// fused append), so that both write the same bytes for the same input.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv.h"

namespace pkv {

// 16 consecutive elements of a row are read in the source type (Src16),
// each divided by the cache's scale (float32, correctly rounded), clamped to
// the largest finite code value and converted in pairs by the hardware
// conversion (round to nearest, ties to even); the 16 codes make one
// 16-byte word (quantize16).  The clamp first makes the conversion
// saturating, as the stored format requires: a value above 448 rounds to 448
// either way, and a NaN passes the clamp and stays NaN.
template <int SRC>
struct Src16;

template <>
struct Src16<PKV_F32> {
  static constexpr int kBytes = 64;
  __device__ static void load(const uint8_t* p, float (&f)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 w = reinterpret_cast<const uint4*>(p)[j];
      f[4 * j] = __uint_as_float(w.x);
      f[4 * j + 1] = __uint_as_float(w.y);
      f[4 * j + 2] = __uint_as_float(w.z);
      f[4 * j + 3] = __uint_as_float(w.w);
    }
  }
};

template <>
struct Src16<PKV_BF16> {
  static constexpr int kBytes = 32;
  __device__ static void load(const uint8_t* p, float (&f)[16]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 w = reinterpret_cast<const uint4*>(p)[j];
      const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[8 * j + 2 * i] = __uint_as_float(x[i] << 16);
        f[8 * j + 2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
      }
    }
  }
};

typedef _Float16 fp8_src_half2_t __attribute__((ext_vector_type(2)));

template <>
struct Src16<PKV_F16> {
  static constexpr int kBytes = 32;
  __device__ static void load(const uint8_t* p, float (&f)[16]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 w = reinterpret_cast<const uint4*>(p)[j];
      const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const fp8_src_half2_t h = __builtin_bit_cast(fp8_src_half2_t, x[i]);
        f[8 * j + 2 * i] = float(h.x);
        f[8 * j + 2 * i + 1] = float(h.y);
      }
    }
  }
};

constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float to_code_range(float x, float scale) {
  const float y = x / scale;
  return y > kE4m3Max ? kE4m3Max : (y < -kE4m3Max ? -kE4m3Max : y);
}

__device__ __forceinline__ uint4 quantize16(const float (&f)[16], float scale) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // bytes 0, 1 from the low-word conversion, bytes 2, 3 from the high
    const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(
        to_code_range(f[4 * j], scale), to_code_range(f[4 * j + 1], scale), 0, false);
    w[j] = __builtin_amdgcn_cvt_pk_fp8_f32(to_code_range(f[4 * j + 2], scale),
                                           to_code_range(f[4 * j + 3], scale), lo, true);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}


}  // namespace pkv
