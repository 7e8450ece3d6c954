// Causal chunked prefill against the paged cache, on gfx950 matrix cores.
//
// What is computed (KV-cache article, intelliparadigm, §2.1 pseudo-code for
// the paged gather and softmax(q K^T) V; §4.1/§4.2 for chunked prefill): a
// chunk of c_b new rows of sequence b, whose K/V are already in the cache
// (n_b tokens cached, chunk included), sits at positions n_b - c_b ..
// n_b - 1; row i attends to positions 0 .. n_b - c_b + i, gathered through
// the block table.
//
// Unlike decode this is a dense contraction (256 query rows share every
// K/V tile), so both products run on MFMA (v_mfma_f32_16x16x32_{bf16,f16}):
//   * one workgroup = 8 wavefronts = 256 query rows of one query head of one
//     sequence; each wavefront owns 32 rows (two 16-row groups);
//   * K/V are walked in tiles of 64 keys.  The workgroup gathers a tile
//     through the block table into LDS -- K and V row-major -- while
//     the previous tile is being computed (the next tile's global loads are
//     in flight during the MFMA work);
//   * S^T = K Q^T (16 keys x 16 rows per MFMA): the accumulator layout puts
//     one query row per lane column and 4 keys per lane, which is exactly
//     the B-operand layout of O^T = V^T P^T once the 8 keys a lane holds
//     for a 32-key step are given consecutive columns of V^T in LDS.  So the
//     online softmax (running max, rescale, sum) needs only two cross-lane
//     steps per row and P never leaves registers;
//   * the PV product runs in float16 whatever the cache's 16-bit type: P is
//     rounded to float16 once (11 significant bits: a weight's relative
//     error is at most 2^-12, so an output row moves by at most 2^-12 of
//     its largest |v|; bfloat16's 8 bits would move rows with a few
//     dominant keys past a 2e-3 tolerance), and a bfloat16 V tile is
//     widened to float16 as it is staged in LDS -- exact for every
//     |v| >= 2^-14 (8 significant bits fit in 11), rounded below that (an
//     error under 2^-25), and limited to |v| <= 65504 as a float16 cache
//     would be.  QK^T stays in the cache type; accumulation and softmax
//     are float32.
// Keys past the causal limit are excluded by select (-inf before exp), and
// keys past the needed range are zero-filled in LDS, so stale or NaN cache
// contents never reach an output.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "common.h"

namespace pkv {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kD = 128;               // head dim served by this kernel
constexpr int kQTile = 32 * kWaves;   // query rows per workgroup
static_assert(kQTile == kPrefillRowsPerGroup, "rows per workgroup");
constexpr int kKTile = 64;            // keys per K/V tile
constexpr int kKRow = kD * 2 + 16;    // LDS bytes per K row (16 B pad)
constexpr int kVRow = kD * 2 + 32;    // LDS bytes per V row (32 B pad)
constexpr int kLdsK = kKTile * kKRow;
constexpr int kLdsV = kKTile * kVRow;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS transpose read (gfx950): every lane reads 8 bytes; within each group
// of 16 lanes, treating lane j's four 16-bit elements as row j of a 16 x 4
// matrix D, lane i receives D[4 k + i / 4][i % 4] for k = 0..3 (checked by
// an in-bounds probe on the GPU).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(const __attribute__((address_space(3))) uint8_t*)(p));
  return __builtin_bit_cast(u32x2, v);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 16-bit element type of the cache: the QK^T MFMA, and how a staged V word
// (two elements) becomes two float16 values.
template <int DT>
struct Half;

// Codes 0, 1 (hi = false) or 2, 3 (hi = true) of a word of E4M3 codes as
// a float16 pair (exact: 3 mantissa bits, exponents within float16's).
__device__ __forceinline__ uint32_t fp8_to_f16x2(uint32_t w, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}

template <>
struct Half<PKV_BF16> {
  // two E4M3 codes as a bfloat16 pair (exact)
  __device__ static uint32_t from_fp8(uint32_t w, bool hi) {
    return __builtin_bit_cast(uint32_t,
                              hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                 : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  }
  __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static uint32_t to_f16x2(uint32_t w) {
    const f32x2 f = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  }
};

template <>
struct Half<PKV_F16> {
  __device__ static uint32_t from_fp8(uint32_t w, bool hi) { return fp8_to_f16x2(w, hi); }
  __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static uint32_t to_f16x2(uint32_t w) { return w; }
};

// O^T += V^T P^T in float16, and two weights as a float16 pair.
__device__ __forceinline__ f32x4 mma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t weights_f16x2(float p0, float p1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, f16x2));
}

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ float fmax_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Lazy rescaling threshold (log2 units): the running max of a row is only
// raised -- and the accumulators rescaled -- when a tile's max exceeds it by
// more than this, so weights stay below 2^8 and the rescale is rare.
constexpr float kRescaleSlack = 8.0f;

// Grid: x = query head (permuted so that heads of one KV group share an
// XCD when num_heads % 8 == 0), y = 256-row tile of the chunk, z = sequence.
// Register use is capped for two waves per SIMD (one eight-wave workgroup
// per CU): one wave's MFMA work then covers the other's waits (measured
// 1.5x over one wave per SIMD at 304 registers).  Eight waves rather than
// two four-wave workgroups share each tile's gather -- its global loads,
// the float16 widening of V and the LDS stores -- and halve the L2 re-reads
// of K/V: 4.8% faster.
//
// K/V tile layout in LDS (two buffers, so one barrier per tile): both
// row-major [64 keys][128 dims], K rows padded to 272 bytes and V rows to
// 288 (float16 V), so that neither the 16-byte K reads of 16 rows nor the
// 8-byte transpose reads of 4 V rows by a 16-lane group share a bank.
// Gather: every thread moves two 16-byte pieces of K and two of V (key
// 32 i + tid / 16, piece tid % 16), 16 consecutive lanes covering one
// contiguous row; a wave's four rows lie in one 16-key group.  The PV product's V^T operand comes out of the row-major
// V tile through the LDS transpose read, so V needs no transposition in
// registers.
// Shared-prefix mode (kPrefix): the rows are the decode queries of a batch
// made of prefix groups -- consecutive rows forked from one parent, whose
// sequences all begin with the group's prefix_len tokens (reached through
// the table of the group's first row).  Every row attends to its group's
// whole prefix -- no causal limit -- and the result is left unnormalised,
// as split-K partials in the first slots of the decode workspace
// ([rows][heads][slots] of head_dim floats, and [rows][heads][slots][2] of
// (max, sum) in log2 units), for the decode merge to combine with the
// private suffixes.  A row tile (blockIdx.y) lies in one group.
struct PrefixArgs {
  float* ws_acc;
  float* ws_ml;
  int32_t* row_info;   // [rows][4]: prefix_len, first row of the group,
                       // prefix slots, 0 (written by split 0 of head 0)
  int32_t slots;       // partials per (row, head) in the workspace
  int32_t split_keys;  // keys per split of a prefix (a multiple of 64):
                       // split z = blockIdx.z takes keys [z, z + 1) *
                       // split_keys of its group's prefix and writes slot z
  int32_t tile_base[kMaxPrefixGroups + 1];  // first row tile of each group
  PrefixGroups groups;
};

// kFp8: the caches hold 8-bit E4M3 codes (DT is the query's type); the
// gather widens each code exactly to DT for K and to float16 for V as it
// stages the tile, so the products are those of the 16-bit path; the K scale
// is in scale_log2 and the V scale (v_scale) multiplies the output rows.
template <int DT, bool kPrefix, bool kFp8 = false>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(
    const uint16_t* __restrict__ query, const uint16_t* __restrict__ key_cache,
    const uint16_t* __restrict__ value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_query_lens,
    int32_t num_heads, int32_t group, int32_t log2_bs, int32_t max_blocks,
    int32_t num_blocks, int32_t total_q, int32_t max_q, float scale_log2,
    float* __restrict__ out, const PrefixArgs pfx, float v_scale = 1.0f) {
  static_assert(!(kFp8 && kPrefix), "8-bit caches: chunked prefill only");
  using H = Half<DT>;
  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][kLdsK];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][kLdsV];

  const int xcd_slice = num_heads >> 3;
  const int h = (num_heads & 7) == 0
                    ? (blockIdx.x & 7) * xcd_slice + (blockIdx.x >> 3)
                    : blockIdx.x;
  // Shared-prefix mode: the row tile's group is the last g whose first
  // tile is at or before blockIdx.y (groups with no rows have no tiles)
  int g = 0;
  if constexpr (kPrefix) {
    int hi = pfx.groups.count - 1;
    while (g < hi) {
      const int mid = (g + hi + 1) >> 1;
      if (pfx.tile_base[mid] <= int(blockIdx.y)) g = mid;
      else hi = mid - 1;
    }
  }
  const int qt = kPrefix ? int(blockIdx.y) - pfx.tile_base[g] : int(blockIdx.y);
  // the group's first row reaches the prefix through its table
  const int b = kPrefix ? pfx.groups.start[g] : blockIdx.z;
  const int split = kPrefix ? blockIdx.z : 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = h / group;
  const int num_kv_heads = num_heads / group;
  const int bs = 1 << log2_bs;

  const int q0 = kPrefix ? pfx.groups.start[g] : cu_query_lens[b];
  const int q1 = kPrefix ? pfx.groups.start[g + 1] : cu_query_lens[b + 1];
  if (q0 < 0 || q1 < q0 || q1 > total_q) return;  // rows unknown: nothing written
  const int c = q1 - q0;
  const int r0 = qt * kQTile;
  if (r0 >= c) return;
  const int n = kPrefix ? pfx.groups.prefix_len[g] : context_lens[b];
  const int rows_here = min(kQTile, c - r0);
  if constexpr (kPrefix) {
    // each row's record for the suffix and merge launches, then only the
    // splits the group's prefix has do work (none for a group with no prefix)
    const int prefix_splits = (n + pfx.split_keys - 1) / pfx.split_keys;
    if (blockIdx.x == 0 && split == 0)
      for (int i = tid; i < rows_here; i += kThreads)
        *reinterpret_cast<int4*>(pfx.row_info + int64_t(q0 + r0 + i) * 4) =
            make_int4(n, q0, prefix_splits, 0);
    if (split >= prefix_splits) return;
  }

  const bool bad_len = kPrefix ? int64_t(n) > (int64_t(max_blocks) << log2_bs)
                               : c > n || c > max_q ||
                                     int64_t(n) > (int64_t(max_blocks) << log2_bs);
  if constexpr (kPrefix) {
    if (bad_len) {  // rows NaN through their prefix partials
      const float nan = __builtin_nanf("");
      for (int i = tid; i < rows_here * kD; i += kThreads) {
        const int64_t row = (int64_t(q0 + r0 + i / kD) * num_heads + h) * pfx.slots + split;
        pfx.ws_acc[row * kD + (i % kD)] = nan;
        if (i % kD == 0) pfx.ws_ml[row * 2] = pfx.ws_ml[row * 2 + 1] = nan;
      }
      return;
    }
  }
  if (bad_len) {
    const float nan = __builtin_nanf("");
    for (int i = tid; i < rows_here * kD; i += kThreads)
      out[(int64_t(q0 + r0 + i / kD) * num_heads + h) * kD + (i % kD)] = nan;
    return;
  }

  const int pos_base = n - c;                    // position of chunk row 0
  // keys [0, kv_end) are needed (the whole prefix in shared-prefix mode)
  const int kv_begin = kPrefix ? split * pfx.split_keys : 0;
  const int kv_end = kPrefix ? min(n, kv_begin + pfx.split_keys) : pos_base + r0 + rows_here;
  const int tile0 = kv_begin / kKTile;  // kv_begin is a multiple of the tile
  const int ntiles = cdiv(kv_end, kKTile);

  // ---- this wavefront's rows ------------------------------------------------
  const int wrows = max(0, min(32, rows_here - 32 * wave));
  const int pos_first = pos_base + r0 + 32 * wave;  // position of its row 0
  // last key any of its rows sees
  const int pos_last = kPrefix ? kv_end - 1 : pos_first + wrows - 1;
  const int col = lane & 15;  // query row within a 16-row group / key within 16
  const int grp = lane >> 4;  // lane group: 8-element k slice, 4-row output slice

  // Q^T as the B operand of S^T = K Q^T: lane holds row (16 qg + col), head
  // dims 32 ks + 8 grp .. + 7.  Rows past the chunk are zero.  A negative
  // scale is applied as an exact sign flip of q, so the softmax below can
  // take maxima of the raw scores and fold |scale| into one FMA.
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const float sl2 = fabsf(scale_log2);
  u32x4 qf[2][kD / 32];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const int i = r0 + 32 * wave + 16 * qg + col;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      if (i < c) {
        qf[qg][ks] = *reinterpret_cast<const u32x4*>(
                         query + (int64_t(q0 + i) * num_heads + h) * kD + 32 * ks + 8 * grp) ^
                     qsign;
      } else {
        qf[qg][ks] = u32x4{0, 0, 0, 0};
      }
    }
  }

  // ---- tile gather ----------------------------------------------------------
  // piece i of this thread: key 16 i + pk of the tile, dims 8 pd .. + 7
  // pieces per thread and tile; a piece row within its 16-key group.
  // 8-bit caches: one piece per thread, key tid / 8 of the tile, dims
  // 16 (tid % 8) .. + 15 (16 codes), widened to two 16-byte LDS pieces.
  constexpr int kPieces = kFp8 ? 1 : kKTile * 16 / kThreads;
  constexpr int kPieceStride = kThreads / 16;  // keys between a thread's pieces
  const int pk = tid >> 4, pd = tid & 15;
  const int64_t tile_elems = int64_t(bs) * kD;
  const int64_t blk_elems = tile_elems * num_kv_heads;
  const int32_t* table = block_tables + int64_t(b) * max_blocks;
  const uint16_t* k_head = key_cache + int64_t(kvh) * tile_elems;
  const uint16_t* v_head = value_cache + int64_t(kvh) * tile_elems;
  const uint32_t lane_elems = uint32_t((pk & 15) * kD + 8 * pd);  // within a 16-key group
  bool bad_blk = false;
  u32x4 gk[kPieces], gv[kPieces];  // the staged 16-byte pieces

  // Loads are unconditional and in bounds.  Blocks hold 16 tokens or more,
  // so the 16 keys of a piece group (16-aligned) share one block: its id is
  // one uniform load per group and tile, and the group's address is a
  // uniform base plus the lane's constant offset.  A group past kv_end
  // re-reads the 16-aligned group holding key kv_end - 1 (a valid row range
  // of a checked block); keys past kv_end, whatever they read, are zeroed
  // when the last, partial tile is stored.
  // 8-bit caches: the key of this thread's piece and its 16 codes' offset
  const int fkey = tid >> 3, fpd = tid & 7;
  const uint8_t* k8_head = reinterpret_cast<const uint8_t*>(key_cache) + int64_t(kvh) * tile_elems;
  const uint8_t* v8_head =
      reinterpret_cast<const uint8_t*>(value_cache) + int64_t(kvh) * tile_elems;
  const uint32_t lane_bytes8 = uint32_t((fkey & 15) * kD + 16 * fpd);  // within a 16-key group
  auto load_tile = [&](int j) {
    const int key0 = j * kKTile;
    if constexpr (kFp8) {
      // the 16-key group of key tid / 8 is 16 (wave / 2): a scalar
      const int gkey = min(key0 + 16 * (wave >> 1), kv_end - 1);
      int id = __builtin_amdgcn_readfirstlane(table[gkey >> log2_bs]);
      if (id < 0 || id >= num_blocks) {
        bad_blk = true;
        id = 0;
      }
      // element offsets are byte offsets for 1-byte codes
      const int64_t grp8 = int64_t(id) * blk_elems + int64_t(gkey & (bs - 1) & ~15) * kD;
      gk[0] = *reinterpret_cast<const u32x4*>(k8_head + grp8 + lane_bytes8);
      gv[0] = *reinterpret_cast<const u32x4*>(v8_head + grp8 + lane_bytes8);
      return;
    }
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      // the piece's 16-key group, 16 (pk >> 4) = 16 (tid >> 8), is the same
      // for all lanes of a wave: taken from the wave index it is a scalar,
      // so the table read and the group's address are scalar work
      const int gkey = min(key0 + kPieceStride * i + 16 * (wave >> 2), kv_end - 1);
      int id = __builtin_amdgcn_readfirstlane(table[gkey >> log2_bs]);
      if (id < 0 || id >= num_blocks) {
        bad_blk = true;
        id = 0;
      }
      const int64_t group = int64_t(id) * blk_elems + int64_t(gkey & (bs - 1) & ~15) * kD;
      gk[i] = *reinterpret_cast<const u32x4*>(k_head + group + lane_elems);
      gv[i] = *reinterpret_cast<const u32x4*>(v_head + group + lane_elems);
    }
  };

  auto store_tile = [&](int buf, int j) {
    const int key0 = j * kKTile;
    if constexpr (kFp8) {
      if (key0 + fkey >= kv_end) gk[0] = gv[0] = u32x4{0, 0, 0, 0};  // code 0 is +0
      u32x4 k2[2], v2[2];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        k2[w / 2][2 * (w % 2)] = H::from_fp8(gk[0][w], false);
        k2[w / 2][2 * (w % 2) + 1] = H::from_fp8(gk[0][w], true);
        v2[w / 2][2 * (w % 2)] = fp8_to_f16x2(gv[0][w], false);
        v2[w / 2][2 * (w % 2) + 1] = fp8_to_f16x2(gv[0][w], true);
      }
      uint8_t* kr = s_k[buf] + fkey * kKRow + 32 * fpd;
      uint8_t* vr = s_v[buf] + fkey * kVRow + 32 * fpd;
      *reinterpret_cast<u32x4*>(kr) = k2[0];
      *reinterpret_cast<u32x4*>(kr + 16) = k2[1];
      *reinterpret_cast<u32x4*>(vr) = v2[0];
      *reinterpret_cast<u32x4*>(vr + 16) = v2[1];
      return;
    }
    if (key0 + kKTile > kv_end) {  // last tile: zero the keys past the range
#pragma unroll
      for (int i = 0; i < kPieces; ++i)
        if (key0 + kPieceStride * i + pk >= kv_end) gk[i] = gv[i] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      *reinterpret_cast<u32x4*>(s_k[buf] + (kPieceStride * i + pk) * kKRow + 16 * pd) = gk[i];
      u32x4 v = gv[i];
#pragma unroll
      for (int w = 0; w < 4; ++w) v[w] = H::to_f16x2(v[w]);  // V as float16
      *reinterpret_cast<u32x4*>(s_v[buf] + (kPieceStride * i + pk) * kVRow + 16 * pd) = v;
    }
  };

  // ---- running softmax state: per lane, rows 16 qg + col -------------------
  f32x4 o[2][kD / 16];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt) o[qg][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};  // log2 units, scale applied
  // Row sums of the float16 weights, on the matrix cores: a ones row in the
  // A operand (dim 0 of a 16-dim tile) against P^T puts each query row's
  // sum in output row 0, i.e. element 0 of lanes 0..15 (lane = query row).
  f32x4 l_acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const uint32_t one_w = col == 0 ? 0x3C003C00u : 0u;  // float16 1.0 pairs
  const u32x4 ones = {one_w, one_w, one_w, one_w};

  auto compute_tile = [&](int buf, int j) {
    const int key0 = j * kKTile;
    const uint8_t* sk = s_k[buf];
    const uint8_t* sv = s_v[buf];
    // S^T tiles: kt = 16-key slice, one per (row group, slice)
    f32x4 s[2][4];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[qg][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            sk + (16 * kt + col) * kKRow + 64 * ks + 16 * grp);
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) s[qg][kt] = H::mma(a, qf[qg][ks], s[qg][kt]);
      }
    }

    // causal limit: only tiles reaching past this wave's first row mask.
    // Key 16 kt + 4 grp + r of the tile is visible to row 16 qg + col iff
    // 16 kt + r <= lim[qg].  Shared-prefix mode: every row sees keys up to
    // n - 1, so only the tile holding the prefix's end masks.
    const bool diag = kPrefix ? key0 + kKTile > kv_end : key0 + kKTile - 1 > pos_first;
    int lim[2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg)
      lim[qg] = kPrefix ? kv_end - 1 - key0 - 4 * grp
                        : pos_first + 16 * qg + col - key0 - 4 * grp;
    if (diag) {
#pragma unroll
      for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kt + r > lim[qg]) s[qg][kt][r] = -INFINITY;
    }

    float mts[2];
    bool grow = false;
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      // NaN-propagating maximum (v_maximum3_f32): unlike fmaxf it needs no
      // quieting pass over the matrix-core results first; a NaN score
      // makes the row NaN either way
      float mt = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        mt = fmax_nan(mt, fmax_nan(fmax_nan(s[qg][kt][0], s[qg][kt][1]),
                                   fmax_nan(s[qg][kt][2], s[qg][kt][3])));
      // across the four lane groups (lane bits 16 and 32): each swap gives
      // both halves of a pair of rows, so the max of the two results is
      // the butterfly step
      const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                        false, false);
      mt = fmax_nan(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
      const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                        false, false);
      mt = fmax_nan(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
      mts[qg] = mt == -INFINITY ? -INFINITY : mt * sl2;  // no -inf * 0
      grow |= mts[qg] > m_run[qg] + kRescaleSlack;
    }
    // a row's max only moves up when it outgrows the slack; every row has
    // key 0, so the first tile always sets it
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        const bool up = mts[qg] > m_run[qg] + kRescaleSlack;
        const float m_new = up ? mts[qg] : m_run[qg];
        const float alpha = __builtin_amdgcn_exp2f(m_run[qg] - m_new);
        m_run[qg] = m_new;
        l_acc[qg] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kD / 16; ++dt) o[qg][dt] *= alpha;
      }
    }
    // P and O^T += V^T P^T one 32-key step at a time: the exp and rounding
    // of step 1 (VALU) then issue while step 0's MFMAs execute, and step 1's
    // MFMAs overlap the next tile's LDS stores; V^T operands stay shared
    // by both row groups.
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      uint32_t pw[2][4];  // [qg][word]: float16 weight pairs
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        const float nm = -m_run[qg];
        float x[8];  // element e = 4 t + r: key 32 st + 16 t + 4 grp + r (slice 2 st + t)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[e] = __builtin_amdgcn_exp2f(fmaf(s[qg][2 * st + (e >> 2)][e & 3], sl2, nm));
        if (diag) {  // masked weights are exactly 0, whatever the scale
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (16 * (2 * st + (e >> 2)) + (e & 3) > lim[qg]) x[e] = 0.f;
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) pw[qg][w] = weights_f16x2(x[2 * w], x[2 * w + 1]);
      }
#pragma unroll
      for (int dt = 0; dt < kD / 16; ++dt) {
        // V^T operand: element e = 4 t + k of lane (grp, col) is dim 16 dt +
        // col of key 32 st + 16 t + 4 grp + k -- the keys this lane's P
        // elements hold.  Transpose read t: lane (grp, col) reads key
        // 32 st + 16 t + 4 grp + col / 4, dims 16 dt + 4 (col % 4) .. + 3.
        const uint8_t* vrow = sv + (32 * st + 4 * grp + (col >> 2)) * kVRow +
                              (16 * dt + 4 * (col & 3)) * 2;
        const u32x2 v0 = lds_read_tr16(vrow);
        const u32x2 v1 = lds_read_tr16(vrow + 16 * kVRow);
        const u32x4 a = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
          const u32x4 bp = {pw[qg][0], pw[qg][1], pw[qg][2], pw[qg][3]};
          o[qg][dt] = mma_f16(a, bp, o[qg][dt]);
        }
      }
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        const u32x4 bp = {pw[qg][0], pw[qg][1], pw[qg][2], pw[qg][3]};
        l_acc[qg] = mma_f16(ones, bp, l_acc[qg]);
      }
    }
  };

  // tile j lives in LDS buffer (j - tile0) % 2; tile j + 1's loads are in
  // flight while tile j is computed, then stored into the other buffer
  // (last read two barriers ago)
  load_tile(tile0);
  store_tile(0, tile0);
  __syncthreads();
  for (int j = tile0; j < ntiles; ++j) {
    if (j + 1 < ntiles) load_tile(j + 1);
    if (wrows > 0 && j * kKTile <= pos_last) compute_tile((j - tile0) & 1, j);
    if (j + 1 < ntiles) store_tile((j + 1 - tile0) & 1, j + 1);
    __syncthreads();
  }
  bad_blk = __syncthreads_or(bad_blk);

  // ---- normalise and store: lane holds rows 16 qg + col, head dims
  // ---- 16 dt + 4 grp .. + 3 ------------------------------------------------
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const float l = __shfl(l_acc[qg][0], col);  // row sum from lane col
    const int i = r0 + 32 * wave + 16 * qg + col;
    if (i >= c) continue;
    if constexpr (kPrefix) {
      // unnormalised partial in the split's slot, with the row's running
      // max (log2 units, the scale applied) and its sum
      const float nan = __builtin_nanf("");
      const int64_t prow = (int64_t(q0 + i) * num_heads + h) * pfx.slots + split;
      float* acc = pfx.ws_acc + prow * kD;
#pragma unroll
      for (int dt = 0; dt < kD / 16; ++dt)
        *reinterpret_cast<f32x4*>(acc + 16 * dt + 4 * grp) =
            bad_blk ? f32x4{nan, nan, nan, nan} : o[qg][dt];
      if (grp == 0) {
        pfx.ws_ml[prow * 2] = bad_blk ? nan : m_run[qg];
        pfx.ws_ml[prow * 2 + 1] = bad_blk ? nan : l;
      }
      continue;
    }
    const float inv = bad_blk ? __builtin_nanf("") : (kFp8 ? v_scale / l : 1.0f / l);
    float* row = out + (int64_t(q0 + i) * num_heads + h) * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt)
      *reinterpret_cast<f32x4*>(row + 16 * dt + 4 * grp) = o[qg][dt] * inv;
  }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

namespace {
// The chunked prefill over 16-bit caches (dtype = the caches' and query's
// type) or over 8-bit caches (fp8: dtype = the query's type, the caches
// E4M3 codes with per-cache scales).
int32_t prefill_call(const void* query, const void* key_cache, const void* value_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* cu_query_lens, int32_t num_seqs, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t max_blocks_per_seq, int32_t num_blocks, int32_t total_query_rows,
                     int32_t max_query_len, float scale, float k_scale, float v_scale,
                     float* out, int32_t dtype, void* stream, bool fp8) {
  if (dtype != PKV_BF16 && dtype != PKV_F16) {
    if (fp8)
      return fail(PKV_ERR_INVALID, "query_dtype %d must be BF16 or F16 for an 8-bit cache",
                  dtype);
    if (dtype_bytes(dtype) == 0) return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
    return fail(PKV_ERR_UNSUPPORTED, "chunked prefill needs a float16 or bfloat16 cache");
  }
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) &&
               v_scale > 0.0f))
    return fail(PKV_ERR_INVALID, "k_scale and v_scale must be positive and finite");
  if (num_seqs < 0 || total_query_rows < 0 || max_query_len < 0)
    return fail(PKV_ERR_INVALID, "negative size");
  if (num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "at most 65535 sequences per call");
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_heads %d must be a positive multiple of num_kv_heads %d",
                num_heads, num_kv_heads);
  if (head_dim != kD)
    return fail(PKV_ERR_UNSUPPORTED, "chunked prefill supports head_dim 128 (got %d)", head_dim);
  if (!is_pow2(block_size) || block_size < 16 || block_size > 256)
    return fail(PKV_ERR_UNSUPPORTED, "block_size must be a power of two in [16, 256]");
  if (max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID, "invalid table/pool sizes");
  if (int64_t(num_blocks) * block_size >= (int64_t(1) << 31))
    return fail(PKV_ERR_INVALID, "num_blocks * block_size must be below 2^31");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "scale must be finite");
  if (num_seqs == 0 || total_query_rows == 0 || max_query_len == 0) return ok();
  if (!query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !cu_query_lens || !out)
    return fail(PKV_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) || !aligned16(out))
    return fail(PKV_ERR_INVALID, "query, caches and out must be 16-byte aligned");
  const int64_t tiles = (int64_t(max_query_len) + kQTile - 1) / kQTile;
  if (tiles > 65535) return fail(PKV_ERR_UNSUPPORTED, "max_query_len too large");
  int log2_bs = 0;
  while ((1 << log2_bs) < block_size) ++log2_bs;
  const float sl2 = (fp8 ? scale * k_scale : scale) * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(num_heads, unsigned(tiles), num_seqs);
  const int group = num_heads / num_kv_heads;
  const auto* q = static_cast<const uint16_t*>(query);
  const auto* kc = static_cast<const uint16_t*>(key_cache);
  const auto* vc = static_cast<const uint16_t*>(value_cache);
#define PKV_PREFILL_LAUNCH(DT, FP8)                                                           \
  hipLaunchKernelGGL((prefill_kernel<DT, false, FP8>), grid, dim3(kThreads), 0, s, q, kc, vc, \
                     block_tables, context_lens, cu_query_lens, num_heads, group, log2_bs,      \
                     max_blocks_per_seq, num_blocks, total_query_rows, max_query_len, sl2, out, \
                     PrefixArgs{}, v_scale)
  if (dtype == PKV_BF16) {
    if (fp8) PKV_PREFILL_LAUNCH(PKV_BF16, true);
    else PKV_PREFILL_LAUNCH(PKV_BF16, false);
  } else {
    if (fp8) PKV_PREFILL_LAUNCH(PKV_F16, true);
    else PKV_PREFILL_LAUNCH(PKV_F16, false);
  }
#undef PKV_PREFILL_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

extern "C" int32_t pkv_paged_attention_prefill(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* cu_query_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t total_query_rows,
    int32_t max_query_len, float scale, float* out, int32_t dtype, void* stream) {
  return prefill_call(query, key_cache, value_cache, block_tables, context_lens, cu_query_lens,
                      num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                      max_blocks_per_seq, num_blocks, total_query_rows, max_query_len, scale,
                      1.0f, 1.0f, out, dtype, stream, false);
}

extern "C" int32_t pkv_paged_attention_prefill_fp8(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* cu_query_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t total_query_rows,
    int32_t max_query_len, float scale, float k_scale, float v_scale, float* out,
    int32_t query_dtype, void* stream) {
  return prefill_call(query, key_cache, value_cache, block_tables, context_lens, cu_query_lens,
                      num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                      max_blocks_per_seq, num_blocks, total_query_rows, max_query_len, scale,
                      k_scale, v_scale, out, query_dtype, stream, true);
}

// The prefix part of the shared-prefix decode: the prefill kernel in
// shared-prefix mode over the decode queries ([rows][num_heads][128]) of
// every group, grid (query head, row tiles of all groups, key ranges).
// Arguments are checked by the caller.
int pkv::launch_prefix_partials(int32_t dtype, const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                const PrefixGroups& groups, int32_t num_heads,
                                int32_t num_kv_heads, int32_t block_size,
                                int32_t max_blocks_per_seq, int32_t num_blocks,
                                int32_t split_keys, int32_t max_splits, float scale,
                                float* ws_acc, float* ws_ml, int32_t* row_info, int32_t slots,
                                void* stream) {
  int log2_bs = 0;
  while ((1 << log2_bs) < block_size) ++log2_bs;
  PrefixArgs pfx{};
  pfx.ws_acc = ws_acc;
  pfx.ws_ml = ws_ml;
  pfx.row_info = row_info;
  pfx.slots = slots;
  pfx.split_keys = split_keys;
  pfx.groups = groups;
  int tiles = 0;
  for (int g = 0; g < groups.count; ++g) {
    pfx.tile_base[g] = tiles;
    tiles += (groups.start[g + 1] - groups.start[g] + kQTile - 1) / kQTile;
  }
  pfx.tile_base[groups.count] = tiles;
  const int32_t rows = groups.start[groups.count];
  if (tiles == 0) return static_cast<int>(hipSuccess);
  const dim3 grid(num_heads, unsigned(tiles), unsigned(std::max(1, max_splits)));
  const int group = num_heads / num_kv_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* q = static_cast<const uint16_t*>(query);
  const auto* kc = static_cast<const uint16_t*>(key_cache);
  const auto* vc = static_cast<const uint16_t*>(value_cache);
  const float sl2 = scale * kLog2e;
  if (dtype == PKV_BF16)
    hipLaunchKernelGGL((prefill_kernel<PKV_BF16, true>), grid, dim3(kThreads), 0, s, q, kc, vc,
                       block_tables, nullptr, nullptr, num_heads, group, log2_bs,
                       max_blocks_per_seq, num_blocks, rows, rows, sl2, nullptr, pfx);
  else
    hipLaunchKernelGGL((prefill_kernel<PKV_F16, true>), grid, dim3(kThreads), 0, s, q, kc, vc,
                       block_tables, nullptr, nullptr, num_heads, group, log2_bs,
                       max_blocks_per_seq, num_blocks, rows, rows, sl2, nullptr, pfx);
  return static_cast<int>(hipGetLastError());
}
