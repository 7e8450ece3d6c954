// Measurement aid: a plain streaming read of device memory, the achievable
// HBM read rate that the decode kernel's fraction of the published peak is
// judged against.  The KV-cache article (intelliparadigm, §2.1) has the
// paged kernel hide the cost of gathering non-contiguous pages; how close
// the decode comes to a contiguous read of the same bytes is what that
// costs on this GPU.
//
// Each workgroup of 4 wavefronts reads 32 KiB spans (8 consecutive 4 KiB
// rows of 16-byte non-temporal loads, all in flight together), grid-stride
// over the buffer -- the same load width, policy and depth the decode
// kernel uses for its K/V.  The values are folded into one word per lane,
// stored only if it matches a constant, so the loads cannot be dropped.
#include <hip/hip_runtime.h>

#include "common.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
