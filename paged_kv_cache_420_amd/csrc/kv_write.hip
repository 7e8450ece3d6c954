// Cache writes on gfx950: slot-mapped append of new K/V rows and whole-block
// copy (the data side of copy-on-write).
//
// Append: KV-cache article (intelliparadigm) §2.1 -- position p of a sequence
// is row p % block_size of physical block table[p / block_size]; the host
// allocator turns that into one flat slot per new token.  Explainer
// (openEuler/CSDN), serving section: each stored token adds one K and one V
// vector to the cache.  Copy: explainer, memory-sharing section -- shared
// blocks are duplicated before a sequence writes into a shared, partly
// filled block.
//
// Both kernels are pure data movement (HBM-bound): every lane moves one
// 16-byte vector, consecutive lanes move consecutive 16-byte pieces of the
// same row, so a wavefront reads and writes whole 1 KiB spans.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "fp8_codes.h"

namespace pkv {
namespace {

// One lane per 16-byte piece of a (token, kv-head) row.
//   key/value   [T][H][row]           row = head_dim * elem bytes
//   caches      [NB][H][BS][row]
__global__ __launch_bounds__(256) void append_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int32_t* __restrict__ slots, int64_t total_pieces,
    int32_t pieces_per_row, int32_t num_kv_heads, int32_t block_size,
    int64_t num_slots) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total_pieces) return;
  int64_t row = i / pieces_per_row;            // (token, head) row index
  int32_t piece = int32_t(i - row * pieces_per_row);
  int64_t token = row / num_kv_heads;
  int32_t head = int32_t(row - token * num_kv_heads);
  int32_t slot = slots[token];
  if (slot < 0 || slot >= num_slots) return;   // skipped row / out of pool
  int32_t blk = slot / block_size;
  int32_t off = slot - blk * block_size;
  int64_t dst = ((int64_t(blk) * num_kv_heads + head) * block_size + off) *
                    pieces_per_row + piece;
  key_cache[dst] = key[i];
  value_cache[dst] = value[i];
}

// Quantising append into an 8-bit (E4M3) cache: one lane per 16 elements
// of a (token, kv-head) row, quantised by quantize16 (fp8_codes.h) into one
// 16-byte store.
template <int SRC>
__global__ __launch_bounds__(256) void append_fp8_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int32_t* __restrict__ slots, int64_t total_pieces,
    int32_t pieces_per_row, int32_t num_kv_heads, int32_t block_size,
    int64_t num_slots, float k_scale, float v_scale) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total_pieces) return;
  int64_t row = i / pieces_per_row;
  int32_t piece = int32_t(i - row * pieces_per_row);
  int64_t token = row / num_kv_heads;
  int32_t head = int32_t(row - token * num_kv_heads);
  int32_t slot = slots[token];
  if (slot < 0 || slot >= num_slots) return;
  int32_t blk = slot / block_size;
  int32_t off = slot - blk * block_size;
  int64_t dst = ((int64_t(blk) * num_kv_heads + head) * block_size + off) *
                    pieces_per_row + piece;
  float f[16];
  Src16<SRC>::load(key + i * Src16<SRC>::kBytes, f);
  key_cache[dst] = quantize16(f, k_scale);
  Src16<SRC>::load(value + i * Src16<SRC>::kBytes, f);
  value_cache[dst] = quantize16(f, v_scale);
}

// grid.y = pair; each lane copies 16-byte pieces of one block, strided.
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
    int32_t num_blocks, int64_t pieces_per_block) {
  int32_t s = src[blockIdx.y];
  int32_t d = dst[blockIdx.y];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  const uint4* ks = key_cache + int64_t(s) * pieces_per_block;
  const uint4* vs = value_cache + int64_t(s) * pieces_per_block;
  uint4* kd = key_cache + int64_t(d) * pieces_per_block;
  uint4* vd = value_cache + int64_t(d) * pieces_per_block;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
       i < pieces_per_block; i += int64_t(gridDim.x) * blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

int32_t check_cache_args(int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks,
                         int32_t dtype) {
  if (dtype_bytes(dtype) == 0)
    return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return fail(PKV_ERR_INVALID,
                "sizes must be positive (kv_heads %d, head_dim %d, "
                "block_size %d, num_blocks %d)",
                num_kv_heads, head_dim, block_size, num_blocks);
  if ((int64_t(head_dim) * dtype_bytes(dtype)) % 16 != 0)
    return fail(PKV_ERR_INVALID,
                "head_dim * element size must be a multiple of 16 bytes");
  if (int64_t(num_blocks) * block_size >= (int64_t(1) << 31))
    return fail(PKV_ERR_INVALID, "num_blocks * block_size must be below 2^31");
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_paged_kv_append(
    const void* key, const void* value, void* key_cache, void* value_cache,
    const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
    void* stream) {
  int32_t st = check_cache_args(num_kv_heads, head_dim, block_size,
                                num_blocks, dtype);
  if (st != PKV_OK) return st;
  if (num_tokens < 0)
    return fail(PKV_ERR_INVALID, "negative num_tokens %d", num_tokens);
  if (num_tokens == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) ||
      !aligned16(value_cache))
    return fail(PKV_ERR_INVALID, "K/V buffers must be 16-byte aligned");
  const int32_t pieces = head_dim * dtype_bytes(dtype) / 16;
  const int64_t total = int64_t(num_tokens) * num_kv_heads * pieces;
  const int64_t blocks = (total + 255) / 256;
  if (blocks >= (int64_t(1) << 31))
    return fail(PKV_ERR_INVALID, "append too large for one launch");
  hipLaunchKernelGGL(append_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(key),
                     static_cast<const uint4*>(value),
                     static_cast<uint4*>(key_cache),
                     static_cast<uint4*>(value_cache), slot_mapping, total,
                     pieces, num_kv_heads, block_size,
                     int64_t(num_blocks) * block_size);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return ok();
}

extern "C" int32_t pkv_copy_blocks(void* key_cache, void* value_cache,
                                   const int32_t* src, const int32_t* dst,
                                   int32_t num_pairs, int32_t num_blocks,
                                   int32_t num_kv_heads, int32_t block_size,
                                   int32_t head_dim, int32_t dtype,
                                   void* stream) {
  int32_t st = check_cache_args(num_kv_heads, head_dim, block_size,
                                num_blocks, dtype);
  if (st != PKV_OK) return st;
  if (num_pairs < 0)
    return fail(PKV_ERR_INVALID, "negative num_pairs %d", num_pairs);
  if (num_pairs == 0) return ok();
  if (!key_cache || !value_cache || !src || !dst)
    return fail(PKV_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(key_cache) || !aligned16(value_cache))
    return fail(PKV_ERR_INVALID, "caches must be 16-byte aligned");
  if (num_pairs > 65535)
    return fail(PKV_ERR_INVALID, "at most 65535 pairs per call");
  const int64_t pieces = int64_t(num_kv_heads) * block_size * head_dim *
                         dtype_bytes(dtype) / 16;
  int64_t gx = (pieces + 255) / 256;
  if (gx > 64) gx = 64;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(gx), unsigned(num_pairs)),
                     dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(key_cache),
                     static_cast<uint4*>(value_cache), src, dst, num_blocks,
                     pieces);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "copy_blocks launch: %s", hipGetErrorString(e));
  return ok();
}

extern "C" int32_t pkv_paged_kv_append_fp8(
    const void* key, const void* value, void* key_cache, void* value_cache,
    const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, float k_scale,
    float v_scale, int32_t src_dtype, void* stream) {
  if (src_dtype != PKV_F32 && src_dtype != PKV_F16 && src_dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID, "src_dtype %d must be F32, F16 or BF16", src_dtype);
  int32_t st = check_cache_args(num_kv_heads, head_dim, block_size, num_blocks,
                                PKV_FP8_E4M3);
  if (st != PKV_OK) return st;
  if (!(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) &&
        v_scale > 0.0f))
    return fail(PKV_ERR_INVALID, "k_scale and v_scale must be positive and finite");
  if (num_tokens < 0)
    return fail(PKV_ERR_INVALID, "negative num_tokens %d", num_tokens);
  if (num_tokens == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) ||
      !aligned16(value_cache))
    return fail(PKV_ERR_INVALID, "K/V buffers must be 16-byte aligned");
  const int32_t pieces = head_dim / 16;
  const int64_t total = int64_t(num_tokens) * num_kv_heads * pieces;
  const int64_t blocks = (total + 255) / 256;
  if (blocks >= (int64_t(1) << 31))
    return fail(PKV_ERR_INVALID, "append too large for one launch");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* k = static_cast<const uint8_t*>(key);
  const auto* v = static_cast<const uint8_t*>(value);
  auto* kc = static_cast<uint4*>(key_cache);
  auto* vc = static_cast<uint4*>(value_cache);
  const int64_t num_slots = int64_t(num_blocks) * block_size;
  if (src_dtype == PKV_F32)
    hipLaunchKernelGGL(append_fp8_kernel<PKV_F32>, dim3(unsigned(blocks)), dim3(256), 0, s, k, v,
                       kc, vc, slot_mapping, total, pieces, num_kv_heads, block_size, num_slots,
                       k_scale, v_scale);
  else if (src_dtype == PKV_F16)
    hipLaunchKernelGGL(append_fp8_kernel<PKV_F16>, dim3(unsigned(blocks)), dim3(256), 0, s, k, v,
                       kc, vc, slot_mapping, total, pieces, num_kv_heads, block_size, num_slots,
                       k_scale, v_scale);
  else
    hipLaunchKernelGGL(append_fp8_kernel<PKV_BF16>, dim3(unsigned(blocks)), dim3(256), 0, s, k,
                       v, kc, vc, slot_mapping, total, pieces, num_kv_heads, block_size,
                       num_slots, k_scale, v_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "fp8 append launch: %s", hipGetErrorString(e));
  return ok();
}

extern "C" int32_t pkv_swap_blocks(const void* src_key_cache, const void* src_value_cache,
                                   void* dst_key_cache, void* dst_value_cache,
                                   const int32_t* src_blocks, const int32_t* dst_blocks,
                                   int32_t num_pairs, int32_t src_num_blocks,
                                   int32_t dst_num_blocks, int64_t block_bytes, void* stream) {
  if (num_pairs < 0) return fail(PKV_ERR_INVALID, "negative num_pairs %d", num_pairs);
  if (num_pairs == 0) return ok();
  if (!src_key_cache || !src_value_cache || !dst_key_cache || !dst_value_cache ||
      !src_blocks || !dst_blocks)
    return fail(PKV_ERR_INVALID, "NULL pointer argument");
  if (block_bytes <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
    return fail(PKV_ERR_INVALID, "sizes must be positive");
  for (int32_t i = 0; i < num_pairs; ++i)
    if (src_blocks[i] < 0 || src_blocks[i] >= src_num_blocks || dst_blocks[i] < 0 ||
        dst_blocks[i] >= dst_num_blocks)
      return fail(PKV_ERR_INVALID, "pair %d (%d -> %d) outside the pools", i, src_blocks[i],
                  dst_blocks[i]);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* sk = static_cast<const uint8_t*>(src_key_cache);
  const auto* sv = static_cast<const uint8_t*>(src_value_cache);
  auto* dk = static_cast<uint8_t*>(dst_key_cache);
  auto* dv = static_cast<uint8_t*>(dst_value_cache);
  // runs of pairs consecutive on both sides move as one copy
  for (int32_t i = 0; i < num_pairs;) {
    int32_t j = i + 1;
    while (j < num_pairs && src_blocks[j] == src_blocks[j - 1] + 1 &&
           dst_blocks[j] == dst_blocks[j - 1] + 1)
      ++j;
    const int64_t off_s = int64_t(src_blocks[i]) * block_bytes;
    const int64_t off_d = int64_t(dst_blocks[i]) * block_bytes;
    const size_t bytes = size_t(j - i) * size_t(block_bytes);
    hipError_t e = hipMemcpyAsync(dk + off_d, sk + off_s, bytes, hipMemcpyDefault, s);
    if (e == hipSuccess) e = hipMemcpyAsync(dv + off_d, sv + off_s, bytes, hipMemcpyDefault, s);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "swap copy: %s", hipGetErrorString(e));
    i = j;
  }
  return ok();
}
