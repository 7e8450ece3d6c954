// Measurement aid: a plain streaming read of device memory, the achievable
// HBM read rate that the decode kernel's fraction of the published peak is
// read against.  The KV-cache article (intelliparadigm, §2.1) has the
// paged kernel hide the cost of gathering non-contiguous pages; how close
// the decode comes to a contiguous read of the same bytes is what that
// costs on this GPU.
//
// Each workgroup of 4 wavefronts reads 32 KiB spans (8 consecutive 4 KiB
// rows of 16-byte non-temporal loads, all in flight together), grid-stride
// over the buffer -- the same load width, policy and depth the decode
// kernel uses for its K/V.  The values are folded into one word per lane,
// stored only if it matches a constant, so the loads cannot be dropped.
//
// Its matrix-core counterpart: a loop of the chunked prefill's product
// instruction (v_mfma_f32_16x16x32_bf16) with operands in registers and
// four independent accumulators per wavefront, no memory traffic -- the
// rate the matrix cores sustain on this GPU at the clock they hold under
// that load, against which the prefill's share of the published peak is
// read.  This file is built with the MFMA accumulators kept in ordinary
// VGPRs, as the prefill kernel has them.
#include <hip/hip_runtime.h>

#include "common.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                                  int64_t n16,
                                                                  uint32_t* __restrict__ sink) {
  constexpr int64_t kSpan = int64_t(kReadThreads) * kReadUnroll;
  uint32_t acc = 0;
  for (int64_t base = int64_t(blockIdx.x) * kSpan; base < n16;
       base += int64_t(gridDim.x) * kSpan) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t i = base + u * kReadThreads + threadIdx.x;
      v[u] = i < n16 ? __builtin_nontemporal_load(buf + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

constexpr int kMatrixThreads = 256;

__global__ __launch_bounds__(kMatrixThreads) void matrix_loop_kernel(int32_t iters,
                                                                    float* __restrict__ sink) {
  // operands that the compiler cannot fold: functions of the lane and the
  // trip count
  const float x = float(threadIdx.x & 7) + float(iters & 1);
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = __bf16(x + float(e));
    b[e] = __bf16(x - float(e));
  }
  f32x4 c0 = {x, 0.f, 0.f, 0.f}, c1 = {0.f, x, 0.f, 0.f}, c2 = {0.f, 0.f, x, 0.f},
        c3 = {0.f, 0.f, 0.f, x};
  for (int32_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
  }
  const f32x4 s = c0 + c1 + c2 + c3;
  const float v = s[0] + s[1] + s[2] + s[3];
  if (v == 1.2345f) sink[0] = v;  // keeps the products live
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_stream_read(const void* buffer, int64_t bytes, int32_t workgroups,
                                   uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return fail(PKV_ERR_INVALID, "bytes must be a multiple of 16");
  if (workgroups <= 0 || workgroups > (1 << 20))
    return fail(PKV_ERR_INVALID, "workgroups must be in [1, 2^20]");
  if (bytes == 0) return ok();
  if (!buffer || !sink) return fail(PKV_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(buffer)) return fail(PKV_ERR_INVALID, "buffer must be 16-byte aligned");
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buffer),
                     bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "stream read launch: %s", hipGetErrorString(e));
  return ok();
}

extern "C" int32_t pkv_matrix_loop(int32_t iters, int32_t workgroups, float* sink, void* stream) {
  if (iters < 0) return fail(PKV_ERR_INVALID, "iters must be non-negative");
  if (workgroups <= 0 || workgroups > (1 << 20))
    return fail(PKV_ERR_INVALID, "workgroups must be in [1, 2^20]");
  if (!sink) return fail(PKV_ERR_INVALID, "NULL pointer argument");
  if (iters == 0) return ok();
  hipLaunchKernelGGL(matrix_loop_kernel, dim3(workgroups), dim3(kMatrixThreads), 0,
                     static_cast<hipStream_t>(stream), iters, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "matrix loop launch: %s", hipGetErrorString(e));
  return ok();
}
