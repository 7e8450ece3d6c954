// PagedAttention decode on gfx950 (CDNA4).
//
// What is computed (KV-cache article, intelliparadigm, §2.1 and its
// pseudo-code): for each sequence b and query head h, gather the sequence's
// keys and values through its block table -- position p lives at row
// p % block_size of physical block block_tables[b][p / block_size] -- and
// return softmax(scale * q K^T) V over all context_lens[b] cached tokens
// (explainer, openEuler/CSDN, serving section: each decode step attends over
// every token before it, its own K/V stored first).  The article names
// prefetching and on-chip staging as the way the kernel hides the scattered
// page accesses; here that becomes: many workgroups per CU with 16-byte
// loads in flight, block ids staged in LDS, and scores/weights in LDS.
//
// Work split (split-K): one workgroup of 4 wavefronts per (kv head,
// sequence, partition of `part` tokens), kv head fastest in the grid.  It
// serves all G = Hq / Hkv query heads that read this kv head, so each K/V
// tile is fetched from HBM once per group (GQA reuse).  Within the
// workgroup:
//   1. block ids of the partition -> LDS (range-checked);
//   2. QK pass: a "unit" is one 16-byte load per lane = 1 KiB per wavefront,
//      covering TPL consecutive tokens of one (block, kv-head) tile (LPT
//      lanes per token row); a chunk is 4 units.  Each lane takes packed
//      dot products of its slice of q with its slice of K, then the LPT
//      lanes of a row reduce them with a transposed butterfly (each step
//      halves the values a lane holds, so the 4*G partial sums end up
//      spread over the lanes instead of replicated); scaled scores -> LDS;
//   3. softmax over the partition in LDS (per-head max, exp2, sum);
//   4. PV pass: same unit walk over V; each lane scales its slice of V by
//      the weight of its token and accumulates G x EPL floats;
//   5. lanes of different token rows and the 4 wavefronts are summed
//      (lane swaps, then LDS) and the partition's result is written either
//      as the final row (one partition) or as (acc, max, sum) partials that
//      decode_reduce_kernel merges with a log-sum-exp.
// 1..8 flop per KV byte against a ~10 flop/B ridge for non-packed fp32 FMAs:
// memory-bound for MHA and close to VALU-bound at G = 8, so no matrix
// cores: the loads and the VALU work per byte are what matter.  Tokens past the context are excluded by select, never by
// multiplying with zero, so stale or NaN cache contents never leak.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "common.h"
#include "fp8_codes.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnitsPerChunk = 4;  // 16-byte loads per lane per chunk
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ---- element traits: packed dot product of a 16-byte q slice with a
// ---- 16-byte K slice, and widening of a 16-byte V slice to floats.
template <int DT>
struct Elem;

template <>
struct Elem<PKV_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerLane = 8;
  static constexpr int kQBytes = 2;      // bytes per query element
  static constexpr bool kQuantised = false;
  using Q = uint4;                          // a lane's slice of one q row
  __device__ static Q load_q(const uint8_t* slice) {
    return *reinterpret_cast<const uint4*>(slice);
  }
  __device__ static float dot(const uint4& q, const uint4& k, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x),
                                          __builtin_bit_cast(bf16x2_t, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y),
                                          __builtin_bit_cast(bf16x2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z),
                                          __builtin_bit_cast(bf16x2_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w),
                                          __builtin_bit_cast(bf16x2_t, k.w), acc, false);
    return acc;
  }
  __device__ static void widen(const uint4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  // Element e of two token rows a and b as a float16 pair (a_e, b_e):
  // widened to float32 (exact), then converted (exact for 2^-14 <= |v| <=
  // 65504: 8 significant bits fit in 11).
  __device__ static void pair_f16(const uint4& a, const uint4& b, uint32_t (&p)[8]) {
    float fa[8], fb[8];
    widen(a, fa);
    widen(b, fb);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      p[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{fa[e], fb[e]}, f16x2_t));
  }
};

template <>
struct Elem<PKV_F16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerLane = 8;
  static constexpr int kQBytes = 2;      // bytes per query element
  static constexpr bool kQuantised = false;
  using Q = uint4;                          // a lane's slice of one q row
  __device__ static Q load_q(const uint8_t* slice) {
    return *reinterpret_cast<const uint4*>(slice);
  }
  __device__ static float dot(const uint4& q, const uint4& k, float acc) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.x),
                                 __builtin_bit_cast(f16x2_t, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.y),
                                 __builtin_bit_cast(f16x2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.z),
                                 __builtin_bit_cast(f16x2_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.w),
                                 __builtin_bit_cast(f16x2_t, k.w), acc, false);
    return acc;
  }
  __device__ static void widen(const uint4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x2_t h = __builtin_bit_cast(f16x2_t, w[i]);
      f[2 * i] = float(h.x);
      f[2 * i + 1] = float(h.y);
    }
  }
  // Element e of two token rows a and b as a float16 pair (a_e, b_e): the
  // halves regrouped, no conversion.
  __device__ static void pair_f16(const uint4& a, const uint4& b, uint32_t (&p)[8]) {
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[2 * i] = (wa[i] & 0xffffu) | (wb[i] << 16);
      p[2 * i + 1] = (wa[i] >> 16) | (wb[i] & 0xffff0000u);
    }
  }
};

template <>
struct Elem<PKV_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerLane = 4;
  static constexpr int kQBytes = 4;      // bytes per query element
  static constexpr bool kQuantised = false;
  using Q = uint4;                          // a lane's slice of one q row
  __device__ static Q load_q(const uint8_t* slice) {
    return *reinterpret_cast<const uint4*>(slice);
  }
  __device__ static float dot(const uint4& q, const uint4& k, float acc) {
    acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    return acc;
  }
  __device__ static void widen(const uint4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};

// ---- 8-bit (E4M3) cache read with a 16-bit query.  A lane's 16-byte slice
// ---- holds 16 codes; each code widens exactly to bf16 / f16 (3 mantissa
// ---- bits, exponents 2^-9 .. 2^8) and to float32 in one conversion per
// ---- pair, so the dot products and the weighted sums see the stored values
// ---- unchanged; the caches' scales are applied outside the loops.
constexpr int kFp8QBf16 = 100;  // template ids, not ABI values
constexpr int kFp8QF16 = 101;

struct Slice32 {
  uint4 lo, hi;  // 16 query elements of 2 bytes
};

template <class Half>
struct ElemFp8 {
  static constexpr int kSrc = Half::kDtype;  // the query's (and new rows') type
  static constexpr int kBytes = 1;
  static constexpr int kPerLane = 16;
  static constexpr int kQBytes = 2;
  static constexpr bool kQuantised = true;
  using Q = Slice32;
  __device__ static Q load_q(const uint8_t* slice) {
    return Q{reinterpret_cast<const uint4*>(slice)[0], reinterpret_cast<const uint4*>(slice)[1]};
  }
  __device__ static float dot(const Q& q, const uint4& k, float acc) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
    const uint32_t qw[8] = {q.lo.x, q.lo.y, q.lo.z, q.lo.w, q.hi.x, q.hi.y, q.hi.z, q.hi.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = Half::dot2(qw[2 * i], Half::widen_pair(kw[i], false), acc);
      acc = Half::dot2(qw[2 * i + 1], Half::widen_pair(kw[i], true), acc);
    }
    return acc;
  }
  __device__ static void widen(const uint4& v, float (&f)[16]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
      const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
      f[4 * i] = a.x;
      f[4 * i + 1] = a.y;
      f[4 * i + 2] = b.x;
      f[4 * i + 3] = b.y;
    }
  }
};

// Codes 0, 1 (hi = false) or 2, 3 (hi = true) of a word as a 16-bit pair,
// and the packed dot product with a pair of query elements.
struct HalfBf16 {
  static constexpr int kDtype = PKV_BF16;
  __device__ static bf16x2_t widen_pair(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  }
  __device__ static float dot2(uint32_t q, bf16x2_t k, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q), k, acc, false);
  }
};

struct HalfF16 {
  static constexpr int kDtype = PKV_F16;
  __device__ static f16x2_t widen_pair(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  }
  __device__ static float dot2(uint32_t q, f16x2_t k, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q), k, acc, false);
  }
};

template <>
struct Elem<kFp8QBf16> : ElemFp8<HalfBf16> {};
template <>
struct Elem<kFp8QF16> : ElemFp8<HalfF16> {};

// ---- cross-lane exchange for the reduction over the lanes of a token row.
// ---- Lane bit M's partner: quad_perm for bits 1 and 2 and row_ror:8 for
// ---- bit 8 flip exactly that bit; row_half_mirror for bit 4 flips bits 4,
// ---- 2 and 1 together (lane l <-> 7 - l in each half row), which the
// ---- register layout of the score reduction allows for.
template <int M>
__device__ __forceinline__ float lane_swap(float x) {
  int v = __float_as_int(x);
  if constexpr (M == 1) {
    v = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    v = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    v = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  } else if constexpr (M == 8) {
    v = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else {
    v = __shfl_xor(v, M);
  }
  return __int_as_float(v);
}

// ---- Score reduction.  A lane holds N = U*G partial dot products, slot
// ---- s = g*U + u (head-major), each over its share of a token row; the
// ---- row's lanes differ in the bits M = kLpt/2 ... 1, reduced from the top.
// ---- While a lane holds more than one value a step halves them (a
// ---- transposed butterfly): each lane keeps one half and adds its
// ---- partner's copy of that half.  The top steps split heads (the upper
// ---- half of the slots is heads G/2.. at the first step, and so on); for
// ---- those a lane always keeps its lower half and sends its upper one,
// ---- which is right because every lane's q registers were loaded with
// ---- its heads XOR-permuted (head_perm below) so that the partner's upper
// ---- half holds the same heads as the lane's lower half -- one DPP add per
// ---- pair and no selects.  The remaining steps split units and pick the
// ---- half with the lane's bit (two selects and an add per pair); once one
// ---- value is left, the steps are plain butterflies.

// Bit of lane `lane` that flips the heads of the step over lane bit M.
// Bit 4's partner also flips bits 2 and 1, so theirs are taken relative to
// bit 4, which keeps them unchanged across that step.
template <int M>
__device__ __forceinline__ int perm_bit(int lane) {
  const int b = (lane & M) ? 1 : 0;
  if constexpr (M >= 4) return b;
  else return b ^ ((lane & 4) ? 1 : 0);
}

// XOR mask applied to the head index of the lane's q registers: the sum of
// the head masks (G/2, G/4, ...) of the head-splitting steps it takes part
// in, each taken when the lane's bit for that step is set.
template <int kLpt, int G, int M = kLpt / 2, int Mask = G / 2>
__device__ __forceinline__ int head_perm(int lane) {
  if constexpr (M >= 1 && Mask >= 1)
    return (perm_bit<M>(lane) ? Mask : 0) + head_perm<kLpt, G, M / 2, Mask / 2>(lane);
  else
    return 0;
}

template <int M, int N, int HeadSteps>
__device__ __forceinline__ void reduce_scores(float* v, int lane) {
  if constexpr (M >= 1) {
    if constexpr (N > 1 && HeadSteps > 0) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) v[i] += lane_swap<M>(v[i + N / 2]);
      reduce_scores<M / 2, N / 2, HeadSteps - 1>(v, lane);
    } else if constexpr (N > 1) {
      const bool hi = (lane & M) != 0;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        float keep = hi ? v[i + N / 2] : v[i];
        float send = hi ? v[i] : v[i + N / 2];
        v[i] = keep + lane_swap<M>(send);
      }
      reduce_scores<M / 2, N / 2, 0>(v, lane);
    } else {
      v[0] += lane_swap<M>(v[0]);
      reduce_scores<M / 2, 1, 0>(v, lane);
    }
  }
}

// Slot offset of a lane's value 0 after reduce_scores: the upper halves it
// kept at the select steps.
template <int M, int N, int HeadSteps>
__device__ __forceinline__ int reduced_slot(int lane) {
  if constexpr (M >= 1 && N > 1) {
    if constexpr (HeadSteps > 0)
      return reduced_slot<M / 2, N / 2, HeadSteps - 1>(lane);
    else
      return ((lane & M) ? N / 2 : 0) + reduced_slot<M / 2, N / 2, 0>(lane);
  } else {
    return 0;
  }
}

// ---- Combine of the weighted sums over the token rows of a wave: the lanes
// ---- of one d-slice differ in the bits kLpt ... 32.  Transposed as well:
// ---- at bits 32 and 16 the swap instructions exchange the upper half of
// ---- one register with the lower half of another (v_permlane32_swap: the
// ---- upper 32 lanes of the first operand with the lower 32 of the second;
// ---- v_permlane16_swap: the odd rows of the first with the even rows of
// ---- the second), so one swap and one add leave lanes with the bit clear
// ---- holding the sum of value i and lanes with it set that of value
// ---- i + N/2.  Below bit 16 a select-and-shuffle step does the same.
template <int M, int Lo, int N>
__device__ __forceinline__ void combine_rows(float* v, int lane) {
  if constexpr (M >= Lo) {
    static_assert(N > 1, "every step must leave a value per lane");
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      if constexpr (M == 32 || M == 16) {
        const auto r = M == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                                  __float_as_uint(v[i + N / 2]),
                                                                  false, false)
                               : __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                                  __float_as_uint(v[i + N / 2]),
                                                                  false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      } else {
        const bool hi = (lane & M) != 0;
        const float keep = hi ? v[i + N / 2] : v[i];
        const float send = hi ? v[i] : v[i + N / 2];
        v[i] = keep + (M == 8 ? lane_swap<8>(send) : __shfl_xor(send, M));
      }
    }
    combine_rows<M / 2, Lo, N / 2>(v, lane);
  }
}

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

template <int DT, int D, int G, int U>
struct Cfg {
  static constexpr int kEs = Elem<DT>::kBytes;
  static constexpr int kEpl = Elem<DT>::kPerLane;     // elements per lane
  static constexpr int kRow = D * kEs;                // bytes per token row
  static constexpr int kLpt = kRow / 16;              // lanes per token row
  static constexpr int kTpl = 64 / kLpt;              // tokens per unit
  static constexpr int kChunkTok = U * kTpl;          // tokens per chunk
  static constexpr int kNv = U * G;                   // partial sums per lane
  // values left per lane after the transposed butterfly, and plain steps
  static constexpr int kLeft = kNv > kLpt ? kNv / kLpt : 1;
  static constexpr int kPlainLog = kNv >= kLpt ? 0 : ilog2(kLpt) - ilog2(kNv);
  static_assert(kRow % 16 == 0 && 64 % kLpt == 0, "row must split across lanes");
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Units of the chunk number `c` of one wavefront, as 16-byte loads: unit u
// covers tokens c*kChunkTok + u*kTpl .. + kTpl-1 of the partition; a lane
// reads at byte offset `lane_off` = (its token within the unit) * row bytes
// + (its 16-byte piece of the row).  A unit never straddles two blocks (a tile holds at least
// the 1 KiB a unit reads), so the unit's address is uniform -- `tiles`, the
// kv head's tile in block 0, plus block and row offsets, all scalar -- and
// each lane adds its constant 32-bit offset.  Units past the last block of
// the partition re-read its last block (always a valid block id) so every
// load is in bounds and the issue is branch-free; the values they bring
// are masked out by the callers.  kStream selects non-temporal loads: when
// every sequence owns its blocks, a decode step reads each cached token
// once, so K/V should stream past the caches rather than evict what is
// reused (+4-8% on batches with private caches).  When blocks are shared
// by several sequences of the batch (a forked prefix), each shared block
// is read once per sequence and the caches serve all reads after the
// first, so the loads keep the default policy (14% faster on 256
// sequences sharing a 1024-token prefix).
template <class C, int U, bool kStream>
__device__ __forceinline__ void issue_chunk(uint4 (&buf)[U], const uint8_t* tiles,
                                            const int* s_blk, int c, int nblk,
                                            int log2_bs, int64_t blk_stride,
                                            uint32_t lane_off) {
  const int bs_mask = (1 << log2_bs) - 1;
  int blk[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int tu = c * C::kChunkTok + u * C::kTpl;
    blk[u] = __builtin_amdgcn_readfirstlane(s_blk[min(tu >> log2_bs, nblk - 1)]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int tu = c * C::kChunkTok + u * C::kTpl;
    const uint8_t* unit = tiles + (int64_t(blk[u]) * blk_stride + (tu & bs_mask) * C::kRow);
    const u32x4* at = reinterpret_cast<const u32x4*>(unit + lane_off);
    u32x4 t;
    if constexpr (kStream) t = __builtin_nontemporal_load(at);
    else t = *at;
    buf[u] = make_uint4(t.x, t.y, t.z, t.w);
  }
  // Keep the loads here, ahead of the computation on the previous chunk
  // that follows: left to itself the scheduler sinks them (with their
  // block-id reads and address arithmetic) into that computation, and a
  // wave then has only one chunk in flight while it computes.
  __builtin_amdgcn_sched_barrier(0);
}

// Everything a decode launch needs, passed by value as the kernel argument.
struct DecodeParams {
  const uint8_t* query;        // [B][Hq][D]
  const uint8_t* key_cache;    // [NB][Hkv][BS][D]
  const uint8_t* value_cache;
  const int32_t* block_tables; // [B][max_blocks]
  int32_t* block_tables_rw;    // the same array, written by step launches
  const int32_t* context_lens; // [B]
  const uint8_t* key_new;      // [B][Hkv][D] or null: fused append
  const uint8_t* value_new;
  float* out;                  // [B][Hq][D]
  float* ws_acc;               // [B][Hq][max_parts][D]  (split-K partials)
  float* ws_ml;                // [B][Hq][max_parts][2]
  int32_t num_kv_heads, log2_bs, max_blocks, num_blocks, max_ctx, part, max_parts;
  int32_t grid_parts;          // partitions per sequence in the grid (<= max_parts)
  float scale_log2;            // scale * log2(e), times the K scale of an 8-bit cache
  float k_scale, v_scale;      // scales of an 8-bit cache (unused otherwise)
  int32_t shared_blocks;       // nonzero: launch the cached-load kernel (shared blocks)
  // Suffix mode (shared-prefix decode), when row_info is set: the launch
  // covers tokens [start, len) of every sequence, start being the prefix
  // length of its group (row_info[4 b]), and writes its partitions as
  // partials from slot slot_base on (the slots before hold the prefix's
  // partials: row_info[4 b + 2] of them).  row_info[4 b + 1] is the first
  // row of the group, whose table reached the prefix.
  const int32_t* row_info;
  int32_t slot_base;
};

// Where a launch gets each sequence's length and which table entries it
// must see changed.  DeviceMeta: lengths from the device array, tables as
// they are in device memory.  StepMeta: per-step metadata passed by value
// in the kernel arguments (no host-to-device copy on the step's critical
// path) -- the lengths, and the table entries this step's appends set,
// which the kernels apply while staging block ids and persist to the
// device table for later launches.  One launch carries the metadata of at
// most kStepRanks sequences and kStepMaxChanges table changes (kernel-
// argument space); a larger batch is served by consecutive launches over
// consecutive ranks of its work order.
constexpr int kStepRanks = 256;
constexpr int kStepMaxChanges = 192;  // per launch

struct DeviceMeta {
  static constexpr bool kHost = false;
  __device__ int len(const DecodeParams& prm, int b, int) const { return prm.context_lens[b]; }
  // grid (kv head, sequence, partition): the rank is the sequence
  __device__ void work(int& b, int& p, int& rank) const {
    b = rank = blockIdx.y;
    p = blockIdx.z;
  }
  // merge grid (query head, sequence)
  __device__ int merge_seq(int y) const { return y; }
  // the block-table row of batch row b
  __device__ int table_row(int b, int) const { return b; }
};

struct StepMeta {
  static constexpr bool kHost = true;
  // Work order: rank r of this launch serves batch row row[r], longest
  // first over the whole batch, so the longest partitions start first and
  // the short ones fill the end of the launch.  With parts_per_rank > 0
  // the grid is (kv head, rank * parts_per_rank + partition, 1): a
  // sequence's partitions are dispatched together, at its rank, instead of
  // every sequence's second partition after all first ones.  0: grid (kv
  // head, rank, partition).
  int32_t lens[kStepRanks];                // by rank
  int32_t change_key[kStepMaxChanges];     // logical block index << 8 | rank
  int32_t change_block[kStepMaxChanges];   // physical block
  // by rank: the batch row (bits 0-15: its query, output and new K/V rows)
  // and the block-table row it reads (bits 16-31: the batch row itself
  // unless the caller keeps the tables in rows of its own)
  uint32_t row[kStepRanks];
  int32_t num_changes;
  int32_t parts_per_rank;
  __device__ int len(const DecodeParams&, int, int rank) const { return lens[rank]; }
  // merge grid (query head, rank): the launch covers only the ranks up to
  // the last sequence that spans two partitions
  __device__ int merge_seq(int y) const { return int(row[y] & 0xFFFFu); }
  __device__ int table_row(int, int rank) const { return int(row[rank] >> 16); }
  __device__ void work(int& b, int& p, int& rank) const {
    if (parts_per_rank > 0) {
      const int y = blockIdx.y;
      rank = y / parts_per_rank;
      p = y % parts_per_rank;
    } else {
      rank = blockIdx.y;
      p = blockIdx.z;
    }
    b = int(row[rank] & 0xFFFFu);
  }
};

// Workgroups per CU the compiler must fit: 16-bit caches with 8 query heads
// per kv head (the GQA layer) are held to 4 (at most 128 VGPRs, 4 waves per
// SIMD), which the kernel, close to VALU-bound, needs more than registers;
// they fit in 114-117 VGPRs with no spill, so the bound is a guard.  Others
// fit 8 unforced.
template <int DT, int G>
constexpr int decode_min_blocks() {
  return (G >= 8 && Elem<DT>::kBytes == 2) ? 4 : 1;
}

// Dynamic LDS: [scores: max(part*G, kWaves*G*D) floats][block ids][m/l].
// kStream: non-temporal K/V loads (blocks private to their sequences).
template <int DT, int D, int G, int U, class Meta, bool kStream>
__global__ __launch_bounds__(kThreads, (decode_min_blocks<DT, G>())) void decode_partition_kernel(
    const DecodeParams prm, const Meta meta) {
  using C = Cfg<DT, D, G, U>;
  using E = Elem<DT>;
  // With 8 query heads per kv head the kernel is bound by VALU issue rather
  // than by HBM, and the weighted sum over V is most of it: there the
  // weights are rounded to float16 (relative error at most 2^-11) and two
  // tokens go through one packed float16 dot product per element and head
  // (v_dot2_f32_f16, float32 accumulation) instead of two float32 FMAs.
  // A bfloat16 V is widened to float16 exactly within +-65504.
  constexpr bool kF16Pv = E::kBytes == 2 && !E::kQuantised && G >= 8 && U % 2 == 0;
  // 16-byte aligned, so a token row of G weights is read with 16-byte loads
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int32_t num_kv_heads = prm.num_kv_heads, log2_bs = prm.log2_bs;
  const int32_t max_blocks = prm.max_blocks, num_blocks = prm.num_blocks;
  const int32_t part = prm.part, max_parts = prm.max_parts;
  const float scale_log2 = prm.scale_log2;

  // Grid (kv head, sequence, partition), kv head fastest: workgroups go to
  // the 8 XCDs round-robin by linear id, so consecutive ids must carry
  // similar work.  Heads of one partition do; partitions of one sequence do
  // not (the last is ragged and most sequences have fewer than the grid's
  // maximum), and putting them fastest would pile every sequence's first
  // partition onto the same XCDs.
  const int kvh = blockIdx.x;
  int b, p_idx, rank;
  meta.work(b, p_idx, rank);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bs = 1 << log2_bs;
  const int num_heads = num_kv_heads * G;

  const int n = meta.len(prm, b, rank);
  const int64_t trow = meta.table_row(b, rank);  // this sequence's block-table row
  const bool suffix = prm.row_info != nullptr;
  const int slot_base = prm.slot_base;
  const int start = suffix ? prm.row_info[4 * int64_t(b)] : 0;
  const bool bad_len =
      n < start || n > prm.max_ctx || int64_t(n) > int64_t(max_blocks) * bs;
  // in suffix mode a sequence with no token past the prefix has no partition
  const int nparts = bad_len ? 1 : suffix ? cdiv(n - start, part) : max(1, cdiv(n, part));
  if (suffix && start > 0 && p_idx == 0 && !bad_len) {
    // Suffix mode: the group's prefix was read through the table of its
    // first row.  A sequence whose own table does not name the same blocks
    // for it is inconsistent input: its first prefix partial's max becomes
    // NaN, so the merge writes a NaN row (first partition of each kv head;
    // the prefix launch that wrote the partial has completed).
    const int32_t* own = prm.block_tables + trow * max_blocks;
    const int32_t* first =
        prm.block_tables + int64_t(prm.row_info[4 * int64_t(b) + 1]) * max_blocks;
    bool differs = false;
    for (int i = int(threadIdx.x); i < (start >> log2_bs); i += kThreads)
      differs |= own[i] != first[i];
    if (__syncthreads_or(differs) && threadIdx.x < G)
      prm.ws_ml[((int64_t(b) * num_kv_heads * G + int64_t(kvh) * G + threadIdx.x) *
                     prm.max_parts) * 2] = __builtin_nanf("");
  }
  if (p_idx >= nparts) return;

  float* out_row = prm.out + (int64_t(b) * num_heads + int64_t(kvh) * G) * D;
  if (bad_len || n == 0) {
    const float fill = bad_len ? __builtin_nanf("") : 0.0f;
    for (int i = tid; i < G * D; i += kThreads) out_row[i] = fill;
    return;
  }

  const int score_floats = max(part * G, kWaves * G * D);
  float* s_score = smem;
  int* s_blk = reinterpret_cast<int*>(smem + score_floats);
  float* s_red = reinterpret_cast<float*>(s_blk + (part >> 3));  // [2][kWaves][G]

  const int p0 = start + p_idx * part;
  const int ntok = min(part, n - p0);
  const int nblk = (ntok + bs - 1) >> log2_bs;
  const int32_t* table = prm.block_tables + trow * max_blocks + (p0 >> log2_bs);
  for (int i = tid; i < nblk; i += kThreads) s_blk[i] = table[i];
  if constexpr (Meta::kHost) {
    // this step's table changes for this sequence and partition: staged,
    // and persisted once (by the kv-head-0 workgroup of the partition)
    __syncthreads();
    const int j0 = p0 >> log2_bs;
    for (int t = tid; t < meta.num_changes; t += kThreads) {
      const int key = meta.change_key[t];
      const int j = (key >> 8) - j0;
      if ((key & 255) == rank && j >= 0 && j < nblk) {
        s_blk[j] = meta.change_block[t];
        if (kvh == 0) prm.block_tables_rw[trow * max_blocks + j0 + j] = meta.change_block[t];
      }
    }
  }
  __syncthreads();
  bool bad_blk = false;
  for (int i = tid; i < nblk; i += kThreads) {
    const int id = s_blk[i];
    if (id < 0 || id >= num_blocks) {
      bad_blk = true;
      s_blk[i] = 0;
    }
  }
  bad_blk = __syncthreads_or(bad_blk);

  const int64_t tile_bytes = int64_t(bs) * C::kRow;           // one (block, head) tile
  const int64_t blk_stride = tile_bytes * num_kv_heads;

  // Fused append: the partition holding the newest position n - 1 stores
  // this step's K/V row for its kv head there before reading the cache
  // (the same bytes a separate slot-mapped append would write).  Only this
  // workgroup reads those two rows in this launch, and the barrier orders
  // its stores before its own loads (workgroup scope: the stores reach this
  // XCD's L2, the loads miss the L1, which starts every launch empty).  No
  // device-scope fence is needed -- on this GPU one writes back the XCD's
  // whole L2.  An 8-bit cache takes the new rows in the query's 16-bit type
  // and quantises each 16-element piece as the quantising append does.
  // (8-bit caches: the step form only)
  if constexpr (!E::kQuantised || Meta::kHost) {
  if (prm.key_new != nullptr && p_idx == nparts - 1) {
    const int pos = n - 1 - p0;  // within the partition
    if (tid < 2 * C::kLpt && !bad_blk) {
      const int id = s_blk[pos >> log2_bs];
      const bool is_v = tid >= C::kLpt;
      const int piece = tid - (is_v ? C::kLpt : 0);
      const int64_t dst = int64_t(id) * blk_stride + int64_t(kvh) * tile_bytes +
                          int64_t(pos & (bs - 1)) * C::kRow + piece * 16;
      const uint8_t* from = is_v ? prm.value_new : prm.key_new;
      uint8_t* to = const_cast<uint8_t*>(is_v ? prm.value_cache : prm.key_cache);
      if constexpr (E::kQuantised) {
        // 16 codes from 16 elements of 2 bytes
        const int64_t src = ((int64_t(b) * num_kv_heads + kvh) * D + piece * 16) * 2;
        float f[16];
        Src16<E::kSrc>::load(from + src, f);
        *reinterpret_cast<uint4*>(to + dst) = quantize16(f, is_v ? prm.v_scale : prm.k_scale);
      } else {
        const int64_t src = (int64_t(b) * num_kv_heads + kvh) * C::kRow + piece * 16;
        *reinterpret_cast<uint4*>(to + dst) = *reinterpret_cast<const uint4*>(from + src);
      }
    }
    __syncthreads();
  }
  }

  // q slices of the G heads: lane covers bytes (lane % LPT) * 16 of the row;
  // register g holds head g ^ hperm (the score reduction's layout).
  const int dl = lane % C::kLpt;
  const int tok_in_unit = lane / C::kLpt;
  const int hperm = head_perm<C::kLpt, G>(lane);
  typename E::Q q[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    q[g] = E::load_q(prm.query +
                     (int64_t(b) * num_heads + int64_t(kvh) * G + (g ^ hperm)) *
                         (D * E::kQBytes) +
                     dl * (C::kEpl * E::kQBytes));

  const uint8_t* kbase = prm.key_cache + int64_t(kvh) * tile_bytes;
  const uint8_t* vbase = prm.value_cache + int64_t(kvh) * tile_bytes;
  const uint32_t lane_off = uint32_t(tok_in_unit * C::kRow + dl * 16);
  const int nchunks = cdiv(ntok, C::kChunkTok);
  // This wave's chunks are wave, wave + kWaves, ...: nj of them.  The walk
  // over them (walk() below) keeps the next chunk's loads in flight while
  // one is computed, in two register buffers (no copies between them).  Its
  // loop runs while two more chunks exist, so every load it issues is
  // needed and one chunk's loads are outstanding at the loop head; the last
  // one or two chunks are computed after it.  The wait before each compute
  // then covers exactly the buffer it reads, and no load re-reads a chunk
  // (with streaming loads such a re-read would come from HBM again).
  const int nj = wave < nchunks ? (nchunks - 1 - wave) / kWaves + 1 : 0;
  auto my_chunk = [&](int j) { return wave + j * kWaves; };
  // 8-bit caches at G = 8 and head_dim 128 hold 128 accumulator floats per
  // lane: there the peeled tail's second copy of the compute costs spills,
  // and the walk keeps one loop whose prefetch past the end re-reads the
  // wave's last chunk instead (192 VGPRs, two waves per SIMD).
  constexpr bool kPeeled = !(E::kQuantised && G >= 8 && D >= 128);
  // The walk's two buffers; `first_issued`: the wave's first chunk is
  // already in flight in `buf0` (the V pass has it loaded during the softmax).
  uint4 buf0[U], buf1[U];
  auto walk = [&](const uint8_t* base, auto&& compute, bool first_issued) {
    if (nj == 0) return;
    if constexpr (!kPeeled) {
      auto clamped = [&](int j) { return my_chunk(min(j, nj - 1)); };
      if (!first_issued)
        issue_chunk<C, U, kStream>(buf0, base, s_blk, clamped(0), nblk, log2_bs, blk_stride,
                                   lane_off);
      for (int j = 0; j < nj; j += 2) {
        issue_chunk<C, U, kStream>(buf1, base, s_blk, clamped(j + 1), nblk, log2_bs, blk_stride,
                                   lane_off);
        compute(buf0, clamped(j));
        issue_chunk<C, U, kStream>(buf0, base, s_blk, clamped(j + 2), nblk, log2_bs, blk_stride,
                                   lane_off);
        if (j + 1 < nj) compute(buf1, clamped(j + 1));
      }
      return;
    }
    if (!first_issued)
      issue_chunk<C, U, kStream>(buf0, base, s_blk, my_chunk(0), nblk, log2_bs, blk_stride,
                                 lane_off);
    int j = 0;
    for (; j + 2 < nj; j += 2) {
      issue_chunk<C, U, kStream>(buf1, base, s_blk, my_chunk(j + 1), nblk, log2_bs, blk_stride,
                                 lane_off);
      compute(buf0, my_chunk(j));
      issue_chunk<C, U, kStream>(buf0, base, s_blk, my_chunk(j + 2), nblk, log2_bs, blk_stride,
                                 lane_off);
      compute(buf1, my_chunk(j + 1));
    }
    if (j + 1 < nj) {
      issue_chunk<C, U, kStream>(buf1, base, s_blk, my_chunk(j + 1), nblk, log2_bs, blk_stride,
                                 lane_off);
      compute(buf0, my_chunk(j));
      compute(buf1, my_chunk(j + 1));
    } else {
      compute(buf0, my_chunk(j));
    }
  };

  // ---- QK pass ------------------------------------------------------------
  // After the reduction a lane's value i is slot slot0 + i: head
  // (slot / U) ^ hperm of unit slot % U.  Lanes that a final plain
  // butterfly left with a copy of a partner's sums do not store.
  constexpr int kHeadSteps = ilog2(G) < ilog2(C::kLpt) ? ilog2(G) : ilog2(C::kLpt);
  const int slot0 = reduced_slot<C::kLpt / 2, C::kNv, kHeadSteps>(lane);
  const bool score_writer = (dl & ((1 << C::kPlainLog) - 1)) == 0;
  auto qk = [&](const uint4 (&k)[U], int c) {
    const int t0 = c * C::kChunkTok;  // relative to p0
    float v[C::kNv];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int u = 0; u < U; ++u) v[g * U + u] = E::dot(q[g], k[u], 0.0f);
    reduce_scores<C::kLpt / 2, C::kNv, kHeadSteps>(v, lane);
    if (score_writer) {
#pragma unroll
      for (int i = 0; i < C::kLeft; ++i) {
        const int slot = slot0 + i;
        const int u = slot % U, g = (slot / U) ^ hperm;
        const int t = t0 + u * C::kTpl + tok_in_unit;
        s_score[t * G + g] = t < ntok ? v[i] * scale_log2 : -INFINITY;
      }
    }
  };
  walk(kbase, qk, false);
  // The V pass's first chunk goes out now, to arrive during the softmax.
  if (nj > 0)
    issue_chunk<C, U, kStream>(buf0, vbase, s_blk, my_chunk(0), nblk, log2_bs, blk_stride, lane_off);
  __syncthreads();

  // ---- softmax over the partition (entries e = t * G + g; a thread only
  // ---- ever sees head tid % G because kThreads is a multiple of G) ----
  const int nent = nchunks * C::kChunkTok * G;
  float mx = -INFINITY;
  for (int e = tid; e < nent; e += kThreads) mx = fmaxf(mx, s_score[e]);
#pragma unroll
  for (int m = G; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
  if (lane < G) s_red[wave * G + lane] = mx;
  __syncthreads();
  const int my_head = tid % G;
  float head_max = s_red[my_head];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) head_max = fmaxf(head_max, s_red[w * G + my_head]);
  float sum = 0.0f;
  // float16 weights (kF16Pv): pair entry q = pi * G + g holds the weights
  // of head g for the tokens ta, tb = ta + kTpl that a lane meets together
  // in units u and u + 1 (pi = c * (U/2) * kTpl + (u/2) * kTpl + lane's
  // token), as one float16 pair, written over the scores in place: ta >= pi,
  // so a pass reads only at or above the words it writes, and the barrier
  // in each round orders its reads before its writes, while later rounds
  // read only above them.  The sum is taken over the rounded weights the
  // product uses.
  uint32_t* s_pw = reinterpret_cast<uint32_t*>(s_score);
  if constexpr (kF16Pv) {
    constexpr int kPairsPerChunk = (U / 2) * C::kTpl;
    const int npe = nent / 2;
    for (int base = 0; base < npe; base += kThreads) {
      const int q = base + tid;
      uint32_t word = 0;
      if (q < npe) {
        const int pi = q / G, g = q % G;
        const int c = pi / kPairsPerChunk, r = pi % kPairsPerChunk;
        const int ta = c * C::kChunkTok + (r / C::kTpl) * 2 * C::kTpl + r % C::kTpl;
        const _Float16 pa = _Float16(__builtin_amdgcn_exp2f(s_score[ta * G + g] - head_max));
        const _Float16 pb =
            _Float16(__builtin_amdgcn_exp2f(s_score[(ta + C::kTpl) * G + g] - head_max));
        sum += float(pa) + float(pb);
        word = __builtin_bit_cast(uint32_t, f16x2_t{pa, pb});
      }
      __syncthreads();
      if (q < npe) s_pw[q] = word;
    }
  } else {
    for (int e = tid; e < nent; e += kThreads) {
      const float p = __builtin_amdgcn_exp2f(s_score[e] - head_max);
      s_score[e] = p;
      sum += p;
    }
  }
#pragma unroll
  for (int m = G; m < 64; m <<= 1) sum += __shfl_xor(sum, m);
  if (lane < G) s_red[kWaves * G + wave * G + lane] = sum;
  __syncthreads();

  // ---- PV pass, same two-buffer walk over V -------------------------------
  float acc[G][C::kEpl];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < C::kEpl; ++e) acc[g][e] = 0.0f;

  // Rows past the partition's last token are zeroed as raw bits (four
  // selects per 16-byte slice, whatever the element type) before they are
  // widened, so stale or NaN cache contents contribute exactly nothing.
  auto pv = [&](const uint4 (&vv)[U], int c) {
    const int t0 = c * C::kChunkTok;
    if constexpr (kF16Pv) {
      // A lane's tokens of units u and u + 1 (kTpl apart) as float16
      // pairs: one packed dot product per element and head covers both.
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        const int ta = t0 + u * C::kTpl + tok_in_unit, tb = ta + C::kTpl;
        const bool la = ta < ntok, lb = tb < ntok;
        const uint4 ra = make_uint4(la ? vv[u].x : 0u, la ? vv[u].y : 0u, la ? vv[u].z : 0u,
                                    la ? vv[u].w : 0u);
        const uint4 rb = make_uint4(lb ? vv[u + 1].x : 0u, lb ? vv[u + 1].y : 0u,
                                    lb ? vv[u + 1].z : 0u, lb ? vv[u + 1].w : 0u);
        uint32_t vp[C::kEpl];
        E::pair_f16(ra, rb, vp);
        const uint32_t* pw = s_pw + ((c * (U / 2) + u / 2) * C::kTpl + tok_in_unit) * G;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const f16x2_t w2 = __builtin_bit_cast(f16x2_t, pw[g]);
#pragma unroll
          for (int e = 0; e < C::kEpl; ++e)
            acc[g][e] = __builtin_amdgcn_fdot2(w2, __builtin_bit_cast(f16x2_t, vp[e]), acc[g][e],
                                               false);
        }
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * C::kTpl + tok_in_unit;
      const bool live = t < ntok;
      const uint4 raw = make_uint4(live ? vv[u].x : 0u, live ? vv[u].y : 0u,
                                   live ? vv[u].z : 0u, live ? vv[u].w : 0u);
      float f[C::kEpl];
      E::widen(raw, f);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = s_score[t * G + g];
#pragma unroll
        for (int e = 0; e < C::kEpl; ++e) acc[g][e] = fmaf(p, f[e], acc[g][e]);
      }
    }
  };
  walk(vbase, pv, true);

  // ---- combine token rows within the wave, then the waves ----------------
  // Each lane ends with kOut of the G * kEpl sums of its d-slice: flat index
  // j = g * kEpl + e from out0 on.
  constexpr int kOut = G * D / 64;
  float* flat = &acc[0][0];
  combine_rows<32, C::kLpt, G * C::kEpl>(flat, lane);
  int out0 = 0;
#pragma unroll
  for (int m = 32, h = G * C::kEpl / 2; m >= C::kLpt; m >>= 1, h >>= 1)
    if (lane & m) out0 += h;
  __syncthreads();  // everyone is done reading weights from s_score
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int j = out0 + i;
    const int g = j / C::kEpl, e = j % C::kEpl;
    s_score[(wave * G + g) * D + dl * C::kEpl + e] = flat[i];
  }
  __syncthreads();

  const float nan = __builtin_nanf("");
  for (int i = tid; i < G * D; i += kThreads) {
    const int g = i / D;
    float a = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      a += s_score[w * G * D + i];
      l += s_red[kWaves * G + w * G + g];
    }
    float m = s_red[g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_red[w * G + g]);
    if constexpr (E::kQuantised) a *= prm.v_scale;
    if (nparts == 1 && !suffix) {
      out_row[i] = bad_blk ? nan : a / l;
    } else {
      const int64_t row =
          (int64_t(b) * num_heads + int64_t(kvh) * G + g) * max_parts + slot_base + p_idx;
      prm.ws_acc[row * D + (i - g * D)] = bad_blk ? nan : a;
      if (i - g * D == 0) {
        prm.ws_ml[row * 2] = bad_blk ? nan : m;
        prm.ws_ml[row * 2 + 1] = bad_blk ? nan : l;
      }
    }
  }
}

// Merge the partitions of one (sequence, head): with per-partition max m_p
// (log2 units), sum l_p and unnormalised acc_p,
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
template <int D, class Meta>
__global__ __launch_bounds__(64) void decode_reduce_kernel(
    const DecodeParams prm, const Meta meta, int32_t num_heads) {
  const int32_t log2_bs = prm.log2_bs, max_blocks = prm.max_blocks, max_ctx = prm.max_ctx;
  const int32_t part = prm.part, max_parts = prm.max_parts;
  const float* __restrict__ ws_acc = prm.ws_acc;
  const float* __restrict__ ws_ml = prm.ws_ml;
  float* __restrict__ out = prm.out;
  const int h = blockIdx.x;
  const int b = meta.merge_seq(blockIdx.y);
  const int n = meta.len(prm, b, blockIdx.y);
  // suffix mode: the prefix's partials in slots [0, pslots), the suffix's
  // from slot_base on
  const bool suffix = prm.row_info != nullptr;
  const int start = suffix ? prm.row_info[4 * int64_t(b)] : 0;
  const int pslots = suffix ? prm.row_info[4 * int64_t(b) + 2] : 0;
  const bool bad_len = n < start || n > max_ctx ||
                       int64_t(n) > (int64_t(max_blocks) << log2_bs);
  if (bad_len) return;
  const int nparts = pslots + cdiv(n - start, part);
  if (nparts <= 1 && !suffix) return;
  float* o = out + (int64_t(b) * num_heads + h) * D;
  if (nparts == 0) {  // a group with no prefix: an empty context
#pragma unroll
    for (int j = 0; j < D / 64; ++j) o[j * 64 + threadIdx.x] = 0.0f;
    return;
  }
  const int64_t row0 = (int64_t(b) * num_heads + h) * max_parts;
  const int skip = prm.slot_base - pslots;  // slots between the two runs
  float big = -INFINITY;
  bool any_nan = false;
  for (int p = 0; p < nparts; ++p) {
    const float m = ws_ml[(row0 + p + (p < pslots ? 0 : skip)) * 2];
    any_nan |= m != m;
    big = fmaxf(big, m);
  }
  float den = 0.0f;
  float num[D / 64];
#pragma unroll
  for (int j = 0; j < D / 64; ++j) num[j] = 0.0f;
  for (int p = 0; p < nparts; ++p) {
    const int64_t slot = row0 + p + (p < pslots ? 0 : skip);
    const float w = __builtin_amdgcn_exp2f(ws_ml[slot * 2] - big);
    den = fmaf(w, ws_ml[slot * 2 + 1], den);
#pragma unroll
    for (int j = 0; j < D / 64; ++j)
      num[j] = fmaf(w, ws_acc[slot * D + j * 64 + threadIdx.x], num[j]);
  }
#pragma unroll
  for (int j = 0; j < D / 64; ++j)
    o[j * 64 + threadIdx.x] = any_nan ? __builtin_nanf("") : num[j] / den;
}

// Longest partition (fewest partials to merge, least per-workgroup setup)
// that still gives the grid about eight workgroups per CU at the longest
// context; shorter ones only for small batches or few heads.  2048-token
// partitions only while no sequence needs more than two: with a long tail
// of long sequences they leave a tail of long workgroups (measured on the
// 13B-shaped batch, contexts up to 5000: 1% slower than 1024; on the
// shared-prefix batch, contexts up to 3084: 5% faster).
int auto_partition(int num_seqs, int num_kv_heads, int max_ctx) {
  int part = max_ctx <= 4096 ? 2048 : 1024;
  while (part > 128 &&
         int64_t(num_seqs) * num_kv_heads * std::max(1, (max_ctx + part - 1) / part) < 2048)
    part /= 2;
  return part;
}

int32_t resolve_partition(int32_t partition_size, int32_t block_size,
                          int32_t num_seqs, int32_t num_kv_heads,
                          int32_t max_ctx, int32_t* part) {
  int32_t p = partition_size == 0 ? auto_partition(num_seqs, num_kv_heads, max_ctx)
                                  : partition_size;
  if (p < 64 || p > 2048 || p % 64 != 0)
    return fail(PKV_ERR_INVALID,
                "partition_size %d must be a multiple of 64 in [64, 2048]",
                partition_size);
  if (p < block_size) p = block_size;  // a partition holds whole blocks
  if (p % block_size != 0)
    return fail(PKV_ERR_INVALID, "partition_size %d is not a multiple of block_size %d",
                p, block_size);
  *part = p;
  return PKV_OK;
}

template <int DT, int D, int G, class Meta>
hipError_t launch_decode(const DecodeParams& prm, const Meta& meta, int B, hipStream_t stream) {
  const int score_floats = std::max(prm.part * G, kWaves * G * D);
  const size_t lds = size_t(score_floats) * 4 + size_t(prm.part >> 3) * 4 +
                     size_t(2 * kWaves * G) * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;  // beyond one CU's LDS
  dim3 grid(prm.num_kv_heads, B, prm.grid_parts);
  Meta m = meta;
  if constexpr (Meta::kHost) {
    // A sequence's partitions consecutive in the grid (when the row count
    // fits the grid's y limit) for long partitions of private caches: a
    // long sequence's later partitions then start with its first instead
    // of closing the launch as a tail of long workgroups (13B-shaped
    // batch, lengths up to 5000 in 2048-token partitions: 7% faster).
    // Partition-major otherwise: with short partitions a late one is a
    // short tail anyway (GQA batch, 512 tokens: 2% faster this way), and
    // with shared blocks every sequence's first partition reads the shared
    // prefix at once, while it is in the caches (2% faster).
    m.parts_per_rank = 0;
    if (prm.grid_parts > 1 && prm.part >= 1024 && !prm.shared_blocks &&
        int64_t(B) * prm.grid_parts <= 65535) {
      m.parts_per_rank = prm.grid_parts;
      grid = dim3(prm.num_kv_heads, B * prm.grid_parts, 1);
    }
  }
  if (prm.shared_blocks)
    hipLaunchKernelGGL((decode_partition_kernel<DT, D, G, kUnitsPerChunk, Meta, false>), grid,
                       dim3(kThreads), lds, stream, prm, m);
  else
    hipLaunchKernelGGL((decode_partition_kernel<DT, D, G, kUnitsPerChunk, Meta, true>), grid,
                       dim3(kThreads), lds, stream, prm, m);
  return hipGetLastError();
}

template <int DT, int D, class Meta>
hipError_t dispatch_group(int G, const DecodeParams& prm, const Meta& meta, int B,
                          hipStream_t s) {
  switch (G) {
    case 1: return launch_decode<DT, D, 1>(prm, meta, B, s);
    case 2: return launch_decode<DT, D, 2>(prm, meta, B, s);
    case 4: return launch_decode<DT, D, 4>(prm, meta, B, s);
    case 8: return launch_decode<DT, D, 8>(prm, meta, B, s);
  }
  return hipErrorInvalidValue;
}

template <class Meta>
hipError_t dispatch_decode(int32_t dtype, int D, int G, const DecodeParams& prm,
                           const Meta& meta, int B, hipStream_t s) {
  switch (dtype) {
    case PKV_BF16:
      return D == 64 ? dispatch_group<PKV_BF16, 64>(G, prm, meta, B, s)
                     : dispatch_group<PKV_BF16, 128>(G, prm, meta, B, s);
    case PKV_F16:
      return D == 64 ? dispatch_group<PKV_F16, 64>(G, prm, meta, B, s)
                     : dispatch_group<PKV_F16, 128>(G, prm, meta, B, s);
    case kFp8QBf16:
      return D == 64 ? dispatch_group<kFp8QBf16, 64>(G, prm, meta, B, s)
                     : dispatch_group<kFp8QBf16, 128>(G, prm, meta, B, s);
    case kFp8QF16:
      return D == 64 ? dispatch_group<kFp8QF16, 64>(G, prm, meta, B, s)
                     : dispatch_group<kFp8QF16, 128>(G, prm, meta, B, s);
    default:
      return D == 64 ? dispatch_group<PKV_F32, 64>(G, prm, meta, B, s)
                     : dispatch_group<PKV_F32, 128>(G, prm, meta, B, s);
  }
}

template <class Meta>
hipError_t launch_merge(const DecodeParams& prm, const Meta& meta, int B, int Hq, int D,
                        hipStream_t s) {
  if (D == 64)
    hipLaunchKernelGGL((decode_reduce_kernel<64, Meta>), dim3(Hq, B), dim3(64), 0, s, prm, meta,
                       Hq);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<128, Meta>), dim3(Hq, B), dim3(64), 0, s, prm,
                       meta, Hq);
  return hipGetLastError();
}

// Workspace (only when some sequence may span two partitions):
//   [acc: B * Hq * max_parts * D floats][(m, l): B * Hq * max_parts * 2 floats]
size_t workspace_bytes(int B, int Hq, int D, int max_parts) {
  if (max_parts <= 1) return 0;
  return size_t(B) * Hq * max_parts * (size_t(D) + 2) * sizeof(float);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_paged_attention_decode_partition_size(
    int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
    int32_t max_context_len, int32_t partition_size, int32_t* resolved) {
  if (!resolved) return fail(PKV_ERR_INVALID, "resolved is NULL");
  if (num_seqs < 0 || num_kv_heads <= 0 || block_size <= 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID, "invalid sizes");
  int32_t part = 0;
  int32_t st = resolve_partition(partition_size, block_size, num_seqs, num_kv_heads,
                                 max_context_len, &part);
  if (st != PKV_OK) return st;
  *resolved = part;
  return ok();
}

extern "C" int32_t pkv_paged_attention_decode_workspace_size(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_context_len, int32_t partition_size, size_t* bytes) {
  if (!bytes) return fail(PKV_ERR_INVALID, "bytes is NULL");
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0)
    return fail(PKV_ERR_INVALID, "invalid sizes");
  int32_t part = 0;
  // block size does not change the partition count unless it exceeds the
  // partition; 1 keeps the size an upper bound for every block size.
  int32_t st = resolve_partition(partition_size, 1, num_seqs, num_kv_heads,
                                 max_context_len, &part);
  if (st != PKV_OK) return st;
  const int max_parts = std::max(1, (max_context_len + part - 1) / part);
  *bytes = workspace_bytes(num_seqs, num_heads, head_dim, max_parts);
  return ok();
}

namespace pkv {
namespace {

// The launches of one step call (see make_step_plan).
struct StepPlan {
  std::vector<StepMeta> chunks;
  std::vector<int32_t> chunk_ranks;    // ranks of each launch
  const int32_t* host_lens = nullptr;  // [num_seqs], batch order
  int32_t num_seqs = 0;
  int32_t ranks(size_t c) const { return chunk_ranks[c]; }
  // ranks of launch c up to the last one whose length exceeds `part`
  int32_t rows_above(size_t c, int32_t part) const {
    int32_t rows = 0;
    for (int32_t r = 0; r < ranks(c); ++r)
      if (chunks[c].lens[r] > part) rows = r + 1;
    return rows;
  }
};

struct DecodeArgs {
  int32_t G = 0, part = 0, max_parts = 0, log2_bs = 0;
  float* ws_acc = nullptr;
  float* ws_ml = nullptr;
};

// Checks every host-visible argument of the decode calls and derives the
// launch geometry.  `need_inputs` is false for the merge stage, which reads
// only lengths, workspace and output.
int32_t prepare_decode(const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size,
                       int32_t max_blocks_per_seq, int32_t num_blocks,
                       int32_t max_context_len, float scale,
                       int32_t partition_size, float* out, void* workspace,
                       size_t workspace_bytes_given, int32_t dtype,
                       bool need_inputs, DecodeArgs* a) {
  if (dtype == kFp8QBf16 || dtype == kFp8QF16) {
    // 8-bit cache, 16-bit query: checked by the *_fp8 entry points
  } else if (dtype == PKV_FP8_E4M3) {
    return fail(PKV_ERR_INVALID,
                "8-bit caches are read by pkv_paged_attention_decode_fp8 (with a 16-bit query)");
  } else if (dtype_bytes(dtype) == 0) {
    return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
  }
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "negative num_seqs");
  if (num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "at most 65535 sequences per call");
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_heads %d must be a positive multiple of num_kv_heads %d",
                num_heads, num_kv_heads);
  a->G = num_heads / num_kv_heads;
  if (a->G != 1 && a->G != 2 && a->G != 4 && a->G != 8)
    return fail(PKV_ERR_UNSUPPORTED, "heads per kv head must be 1, 2, 4 or 8 (got %d)", a->G);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (!is_pow2(block_size) || block_size < 8 || block_size > 256)
    return fail(PKV_ERR_UNSUPPORTED, "block_size must be a power of two in [8, 256]");
  // a wavefront's 16-byte loads cover 1 KiB of one (block, kv-head) tile:
  // the tile must hold at least that much
  const int cache_elem = (dtype == kFp8QBf16 || dtype == kFp8QF16) ? 1 : dtype_bytes(dtype);
  if (need_inputs && int64_t(block_size) * head_dim * cache_elem < 1024)
    return fail(PKV_ERR_UNSUPPORTED,
                "block_size * head_dim * element size must be at least 1024 bytes (got %d x %d x %d)",
                block_size, head_dim, cache_elem);
  if (max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID, "invalid table/pool sizes");
  if (int64_t(num_blocks) * block_size >= (int64_t(1) << 31))
    return fail(PKV_ERR_INVALID, "num_blocks * block_size must be below 2^31");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "scale must be finite");
  if (num_seqs > 0) {
    if (!context_lens || !out) return fail(PKV_ERR_INVALID, "NULL pointer argument");
    if (need_inputs && (!query || !key_cache || !value_cache || !block_tables))
      return fail(PKV_ERR_INVALID, "NULL pointer argument");
    if (need_inputs && (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache)))
      return fail(PKV_ERR_INVALID, "query and caches must be 16-byte aligned");
    if (!aligned16(out)) return fail(PKV_ERR_INVALID, "out must be 16-byte aligned");
  }
  int32_t st = resolve_partition(partition_size, block_size, num_seqs, num_kv_heads,
                                 max_context_len, &a->part);
  if (st != PKV_OK) return st;
  a->max_parts = std::max(1, (max_context_len + a->part - 1) / a->part);
  if (a->max_parts > 65535) return fail(PKV_ERR_UNSUPPORTED, "context too long");
  const size_t need = workspace_bytes(num_seqs, num_heads, head_dim, a->max_parts);
  if (need > 0 && (!workspace || workspace_bytes_given < need))
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes_given : size_t(0));
  if (need > 0 && !aligned16(workspace))
    return fail(PKV_ERR_INVALID, "workspace must be 16-byte aligned");
  if (need > 0) {
    a->ws_acc = static_cast<float*>(workspace);
    a->ws_ml = a->ws_acc + size_t(num_seqs) * num_heads * a->max_parts * head_dim;
  }
  a->log2_bs = 0;
  while ((1 << a->log2_bs) < block_size) ++a->log2_bs;
  return PKV_OK;
}

// The partition kernel (with the fused append when key_new/value_new are
// given), then -- when `merge` is set and some sequence can span two
// partitions -- the log-sum-exp merge.  The merge is a launch of its own:
// partitions of one sequence run on different XCDs, whose L2s are only
// made coherent with each other at a kernel boundary (a device-scope fence
// per workgroup writes back the whole L2 and costs more than the launch).
// `step` (may be null): lengths and table changes by value, for the step
// calls, one launch per chunk of ranks; context_lens is then unused.
int32_t run_decode(const void* query, const void* key_new, const void* value_new,
                   const void* key_cache, const void* value_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                   int32_t num_blocks, int32_t max_context_len, float scale,
                   int32_t partition_size, float* out, void* workspace,
                   size_t workspace_bytes_given, int32_t dtype, void* stream, bool partials,
                   bool merge, const StepPlan* step, float k_scale = 1.0f,
                   float v_scale = 1.0f) {
  const bool shared_blocks = (dtype & PKV_DECODE_SHARED_BLOCKS) != 0;
  dtype &= ~int32_t(PKV_DECODE_SHARED_BLOCKS);
  DecodeArgs a;
  // the step calls' host lengths were checked when the plan was made
  const int32_t* lens_check = step ? step->host_lens : context_lens;
  int32_t st = prepare_decode(query, key_cache, value_cache, block_tables, lens_check,
                              num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                              max_blocks_per_seq, num_blocks, max_context_len, scale,
                              partition_size, out, workspace, workspace_bytes_given, dtype,
                              partials, &a);
  if (st != PKV_OK) return st;
  if (key_new || value_new) {
    if (!key_new || !value_new) return fail(PKV_ERR_INVALID, "key and value must both be given");
    if (!aligned16(key_new) || !aligned16(value_new))
      return fail(PKV_ERR_INVALID, "key and value must be 16-byte aligned");
  }
  if (num_seqs == 0) return ok();
  DecodeParams prm{};
  prm.query = static_cast<const uint8_t*>(query);
  prm.key_cache = static_cast<const uint8_t*>(key_cache);
  prm.value_cache = static_cast<const uint8_t*>(value_cache);
  prm.block_tables = block_tables;
  prm.block_tables_rw = const_cast<int32_t*>(block_tables);
  prm.context_lens = context_lens;
  prm.key_new = static_cast<const uint8_t*>(key_new);
  prm.value_new = static_cast<const uint8_t*>(value_new);
  prm.out = out;
  prm.ws_acc = a.ws_acc;
  prm.ws_ml = a.ws_ml;
  prm.num_kv_heads = num_kv_heads;
  prm.log2_bs = a.log2_bs;
  prm.max_blocks = max_blocks_per_seq;
  prm.num_blocks = num_blocks;
  prm.max_ctx = max_context_len;
  prm.part = a.part;
  prm.max_parts = a.max_parts;
  prm.grid_parts = a.max_parts;
  prm.scale_log2 = k_scale == 1.0f ? scale * kLog2e : (scale * k_scale) * kLog2e;
  prm.k_scale = k_scale;
  prm.v_scale = v_scale;
  prm.shared_blocks = shared_blocks ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (partials) {
    if (step) {
      for (size_t c = 0; c < step->chunks.size() && e == hipSuccess; ++c)
        e = dispatch_decode(dtype, head_dim, a.G, prm, step->chunks[c], step->ranks(c), s);
    } else {
      e = dispatch_decode(dtype, head_dim, a.G, prm, DeviceMeta{}, num_seqs, s);
    }
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  }
  if (!merge || a.max_parts <= 1) return ok();
  if (step) {
    // the step's lengths are known here: in each launch the merge covers
    // the ranks up to the last sequence that spans two partitions (the
    // order is longest first, so these are the leading ranks); when every
    // sequence fits one partition the partition kernel wrote the final
    // rows and no merge runs
    for (size_t c = 0; c < step->chunks.size() && e == hipSuccess; ++c) {
      const int32_t rows = step->rows_above(c, a.part);
      if (rows > 0) e = launch_merge(prm, step->chunks[c], rows, num_heads, head_dim, s);
    }
  } else {
    e = launch_merge(prm, DeviceMeta{}, num_seqs, num_heads, head_dim, s);
  }
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode merge launch: %s", hipGetErrorString(e));
  return ok();
}

// Makes a step's launch metadata from its host lengths and table changes:
// the work order over the whole batch, cut into launches of at most
// kStepRanks ranks and kStepMaxChanges changes, each carrying its ranks'
// lengths, batch and table rows, and the changes of their rows.
// table_rows (may be null: the batch rows themselves) maps batch row b to
// the block-table row it reads and whose changes it persists.
int32_t make_step_plan(const int32_t* context_lens, const int32_t* changes,
                       int32_t num_changes, int32_t num_seqs, int32_t num_kv_heads,
                       int32_t max_blocks_per_seq, StepPlan* plan,
                       const int32_t* skipped = nullptr, const int32_t* table_rows = nullptr) {
  if (num_seqs > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "at most 65535 sequences per call (got %d)", num_seqs);
  if (num_changes < 0) return fail(PKV_ERR_INVALID, "negative num_changes");
  if (num_seqs > 0 && !context_lens) return fail(PKV_ERR_INVALID, "context_lens is NULL");
  if (num_changes > 0 && !changes) return fail(PKV_ERR_INVALID, "changes is NULL");
  plan->host_lens = context_lens;
  // Longest first (stable), so long partitions start first -- by the tokens
  // the launch reads, the length less the shared prefix (skipped[i]) in a
  // shared-prefix step; then, within each round of R = 256 / num_kv_heads
  // sequences -- the sequences whose workgroups one pass of the dispatcher
  // spreads over all 256 CUs -- every other round reversed ("snake"), so
  // the CUs that get a round's longest sequence get the next round's
  // shortest and the CUs' loads even out when the whole grid is resident at
  // once (7B-shaped batch: partition kernel 1% faster than plain
  // longest-first).
  std::vector<int32_t> idx(num_seqs), order(num_seqs), rank_of(num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) idx[i] = i;
  auto work = [&](int32_t i) {
    return int64_t(context_lens[i]) - (skipped ? skipped[i] : 0);
  };
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return work(a) > work(b); });
  const int32_t R = std::max(1, 256 / std::max(1, num_kv_heads));
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t k = i / R, j = i % R;
    int32_t src = k % 2 == 0 ? i : k * R + (R - 1 - j);
    if (src >= num_seqs) src = i;  // a short last round keeps its order
    order[i] = idx[src];
    rank_of[idx[src]] = i;
  }
  std::vector<int32_t> per_row(num_seqs, 0);
  for (int32_t i = 0; i < num_changes; ++i) {
    const int32_t row = changes[3 * i], blk = changes[3 * i + 1];
    if (row < 0 || row >= num_seqs || blk < 0 || blk >= max_blocks_per_seq || blk >= (1 << 23))
      return fail(PKV_ERR_INVALID, "table change %d (row %d, index %d) out of range", i, row,
                  blk);
    if (++per_row[row] > kStepMaxChanges)
      return fail(PKV_ERR_UNSUPPORTED, "step calls take at most %d table changes per sequence",
                  kStepMaxChanges);
  }
  // launches: consecutive ranks, a new one when the ranks or the changes
  // would not fit
  std::vector<int32_t> chunk_of(num_seqs);
  plan->num_seqs = num_seqs;
  plan->chunks.clear();
  plan->chunk_ranks.clear();
  int32_t in_chunk = 0, changes_in_chunk = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t b = order[i];
    if (plan->chunks.empty() || in_chunk == kStepRanks ||
        changes_in_chunk + per_row[b] > kStepMaxChanges) {
      plan->chunks.emplace_back();
      plan->chunk_ranks.push_back(0);
      in_chunk = changes_in_chunk = 0;
    }
    StepMeta& m = plan->chunks.back();
    const uint32_t trow = table_rows ? uint32_t(table_rows[b]) : uint32_t(b);
    m.lens[in_chunk] = context_lens[b];
    m.row[in_chunk] = uint32_t(b) | (trow << 16);
    chunk_of[b] = int32_t(plan->chunks.size()) - 1;
    rank_of[b] = in_chunk;  // now the rank within its launch
    ++in_chunk;
    ++plan->chunk_ranks.back();
    changes_in_chunk += per_row[b];
  }
  for (int32_t i = 0; i < num_changes; ++i) {
    const int32_t row = changes[3 * i], blk = changes[3 * i + 1];
    StepMeta& m = plan->chunks[chunk_of[row]];
    m.change_key[m.num_changes] = (blk << 8) | rank_of[row];
    m.change_block[m.num_changes] = changes[3 * i + 2];
    ++m.num_changes;
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int32_t pkv_paged_attention_decode_partials(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, float* out, void* workspace,
    size_t workspace_bytes_given, int32_t dtype, void* stream) {
  return run_decode(query, nullptr, nullptr, key_cache, value_cache, block_tables,
                    context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size,
                    out, workspace, workspace_bytes_given, dtype, stream, true, false, nullptr);
}

extern "C" int32_t pkv_paged_attention_decode_merge(
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t partition_size, float* out, void* workspace,
    size_t workspace_bytes_given, void* stream) {
  return run_decode(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, context_lens, num_seqs,
                    num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, 1,
                    max_context_len, 1.0f, partition_size, out, workspace,
                    workspace_bytes_given, PKV_F32, stream, false, true, nullptr);
}

extern "C" int32_t pkv_paged_attention_decode(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, float* out, void* workspace,
    size_t workspace_bytes_given, int32_t dtype, void* stream) {
  return run_decode(query, nullptr, nullptr, key_cache, value_cache, block_tables,
                    context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size,
                    out, workspace, workspace_bytes_given, dtype, stream, true, true, nullptr);
}

extern "C" int32_t pkv_paged_attention_decode_append(
    const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, float* out,
    void* workspace, size_t workspace_bytes_given, int32_t dtype, void* stream) {
  if (num_seqs > 0 && (!key || !value))
    return fail(PKV_ERR_INVALID, "NULL pointer argument");
  return run_decode(query, key, value, key_cache, value_cache, block_tables, context_lens,
                    num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size,
                    out, workspace, workspace_bytes_given, dtype, stream, true, true, nullptr);
}

extern "C" int32_t pkv_paged_attention_decode_append_partials(
    const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, float* out,
    void* workspace, size_t workspace_bytes_given, int32_t dtype, void* stream) {
  if (num_seqs > 0 && (!key || !value))
    return fail(PKV_ERR_INVALID, "NULL pointer argument");
  return run_decode(query, key, value, key_cache, value_cache, block_tables, context_lens,
                    num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size,
                    out, workspace, workspace_bytes_given, dtype, stream, true, false, nullptr);
}

namespace {
int32_t step_call(const void* query, const void* key, const void* value, void* key_cache,
                  void* value_cache, int32_t* block_tables, const int32_t* context_lens,
                  const int32_t* changes, int32_t num_changes, int32_t num_seqs,
                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                  int32_t max_context_len, float scale, int32_t partition_size, float* out,
                  void* workspace, size_t workspace_bytes_given, int32_t dtype, void* stream,
                  bool partials, bool merge) {
  StepPlan plan;
  int32_t st = make_step_plan(context_lens, changes, num_changes, num_seqs, num_kv_heads,
                              max_blocks_per_seq, &plan);
  if (st != PKV_OK) return st;
  return run_decode(query, key, value, key_cache, value_cache, block_tables, nullptr, num_seqs,
                    num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                    num_blocks, max_context_len, scale, partition_size, out, workspace,
                    workspace_bytes_given, dtype, stream, partials, merge, &plan);
}
}  // namespace

extern "C" int32_t pkv_paged_attention_decode_step(
    const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, int32_t* block_tables, const int32_t* context_lens,
    const int32_t* changes, int32_t num_changes, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t num_blocks, int32_t max_context_len, float scale, int32_t partition_size,
    float* out, void* workspace, size_t workspace_bytes_given, int32_t dtype, void* stream) {
  return step_call(query, key, value, key_cache, value_cache, block_tables, context_lens,
                   changes, num_changes, num_seqs, num_heads, num_kv_heads, head_dim,
                   block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                   partition_size, out, workspace, workspace_bytes_given, dtype, stream, true,
                   true);
}

extern "C" int32_t pkv_paged_attention_decode_step_mapped(
    const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, int32_t* block_tables, int32_t num_table_rows,
    const int32_t* table_rows, const int32_t* context_lens, const int32_t* changes,
    int32_t num_changes, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, float* out, void* workspace,
    size_t workspace_bytes_given, int32_t dtype, void* stream) {
  if (num_table_rows < 0 || num_table_rows > 65536)
    return fail(PKV_ERR_INVALID, "num_table_rows %d must be in [0, 65536]", num_table_rows);
  if (num_seqs > 0 && !table_rows) return fail(PKV_ERR_INVALID, "table_rows is NULL");
  if (num_seqs > num_table_rows)
    return fail(PKV_ERR_INVALID, "%d sequences cannot have distinct rows among %d", num_seqs,
                num_table_rows);
  // distinct rows: two sequences persisting changes into one row would race
  std::vector<bool> used(size_t(std::max(num_table_rows, 0)), false);
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t r = table_rows[b];
    if (r < 0 || r >= num_table_rows || used[r])
      return fail(PKV_ERR_INVALID, "table_rows[%d] = %d is out of range or repeated", b, r);
    used[r] = true;
  }
  StepPlan plan;
  int32_t st = make_step_plan(context_lens, changes, num_changes, num_seqs, num_kv_heads,
                              max_blocks_per_seq, &plan, nullptr, table_rows);
  if (st != PKV_OK) return st;
  return run_decode(query, key, value, key_cache, value_cache, block_tables, nullptr, num_seqs,
                    num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                    num_blocks, max_context_len, scale, partition_size, out, workspace,
                    workspace_bytes_given, dtype, stream, true, true, &plan);
}

extern "C" int32_t pkv_paged_attention_decode_step_partials(
    const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, int32_t* block_tables, const int32_t* context_lens,
    const int32_t* changes, int32_t num_changes, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t num_blocks, int32_t max_context_len, float scale, int32_t partition_size,
    float* out, void* workspace, size_t workspace_bytes_given, int32_t dtype, void* stream) {
  return step_call(query, key, value, key_cache, value_cache, block_tables, context_lens,
                   changes, num_changes, num_seqs, num_heads, num_kv_heads, head_dim,
                   block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                   partition_size, out, workspace, workspace_bytes_given, dtype, stream, true,
                   false);
}

extern "C" int32_t pkv_paged_attention_decode_step_merge(
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t partition_size, float* out, void* workspace, size_t workspace_bytes_given,
    void* stream) {
  StepPlan plan;
  int32_t st = make_step_plan(context_lens, nullptr, 0, num_seqs, num_kv_heads,
                              max_blocks_per_seq, &plan);
  if (st != PKV_OK) return st;
  return run_decode(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, num_seqs,
                    num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, 1,
                    max_context_len, 1.0f, partition_size, out, workspace,
                    workspace_bytes_given, PKV_F32, stream, false, true, &plan);
}

namespace {
int32_t fp8_call(const void* query, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                 int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                 int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
                 float scale, float k_scale, float v_scale, int32_t partition_size, float* out,
                 void* workspace, size_t workspace_bytes_given, int32_t query_dtype,
                 void* stream, bool merge, const void* key_new = nullptr,
                 const void* value_new = nullptr, const StepPlan* step = nullptr) {
  const int32_t hint = query_dtype & int32_t(PKV_DECODE_SHARED_BLOCKS);
  query_dtype &= ~int32_t(PKV_DECODE_SHARED_BLOCKS);
  if (query_dtype != PKV_BF16 && query_dtype != PKV_F16)
    return fail(PKV_ERR_INVALID, "query_dtype %d must be BF16 or F16 for an 8-bit cache",
                query_dtype);
  if (!(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
    return fail(PKV_ERR_INVALID, "k_scale and v_scale must be positive and finite");
  return run_decode(query, key_new, value_new, key_cache, value_cache, block_tables,
                    context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size,
                    out, workspace, workspace_bytes_given,
                    (query_dtype == PKV_BF16 ? kFp8QBf16 : kFp8QF16) | hint, stream, true, merge,
                    step, k_scale, v_scale);
}
}  // namespace

extern "C" int32_t pkv_paged_attention_decode_fp8_step(
    const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, int32_t* block_tables, const int32_t* context_lens,
    const int32_t* changes, int32_t num_changes, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t num_blocks, int32_t max_context_len, float scale, float k_scale, float v_scale,
    int32_t partition_size, float* out, void* workspace, size_t workspace_bytes_given,
    int32_t query_dtype, void* stream) {
  StepPlan plan;
  int32_t st = make_step_plan(context_lens, changes, num_changes, num_seqs, num_kv_heads,
                              max_blocks_per_seq, &plan);
  if (st != PKV_OK) return st;
  return fp8_call(query, key_cache, value_cache, block_tables, nullptr, num_seqs, num_heads,
                  num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                  max_context_len, scale, k_scale, v_scale, partition_size, out, workspace,
                  workspace_bytes_given, query_dtype, stream, true, key, value, &plan);
}

extern "C" int32_t pkv_paged_attention_decode_fp8(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, float scale,
    float k_scale, float v_scale, int32_t partition_size, float* out, void* workspace,
    size_t workspace_bytes_given, int32_t query_dtype, void* stream) {
  return fp8_call(query, key_cache, value_cache, block_tables, context_lens, num_seqs,
                  num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                  num_blocks, max_context_len, scale, k_scale, v_scale, partition_size, out,
                  workspace, workspace_bytes_given, query_dtype, stream, true);
}

extern "C" int32_t pkv_paged_attention_decode_fp8_partials(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, float scale,
    float k_scale, float v_scale, int32_t partition_size, float* out, void* workspace,
    size_t workspace_bytes_given, int32_t query_dtype, void* stream) {
  return fp8_call(query, key_cache, value_cache, block_tables, context_lens, num_seqs,
                  num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                  num_blocks, max_context_len, scale, k_scale, v_scale, partition_size, out,
                  workspace, workspace_bytes_given, query_dtype, stream, false);
}

// ---- decode with prefixes shared by groups of sequences -------------------

namespace {
// Checks the host arrays describing the prefix groups and copies them into
// `out`: group g is rows [group_starts[g], group_starts[g + 1]), sharing
// prefix_lens[g] tokens (0, or a multiple of block_size up to
// max_context_len).
int32_t read_groups(int32_t num_seqs, int32_t num_groups, const int32_t* group_starts,
                    const int32_t* prefix_lens, int32_t block_size, int32_t max_context_len,
                    PrefixGroups* out) {
  if (!is_pow2(block_size) || block_size < 16 || block_size > 256)
    return fail(PKV_ERR_UNSUPPORTED, "block_size must be a power of two in [16, 256]");
  if (num_groups < 1) return fail(PKV_ERR_INVALID, "num_groups %d must be positive", num_groups);
  if (num_groups > kMaxPrefixGroups)
    return fail(PKV_ERR_UNSUPPORTED, "at most %d prefix groups per call (got %d)",
                kMaxPrefixGroups, num_groups);
  if (!group_starts || !prefix_lens) return fail(PKV_ERR_INVALID, "NULL group array");
  if (group_starts[0] != 0 || group_starts[num_groups] != num_seqs)
    return fail(PKV_ERR_INVALID, "group_starts must run from 0 to num_seqs %d", num_seqs);
  out->count = num_groups;
  for (int32_t g = 0; g <= num_groups; ++g) {
    if (g > 0 && group_starts[g] < group_starts[g - 1])
      return fail(PKV_ERR_INVALID, "group_starts must not decrease (group %d)", g - 1);
    out->start[g] = group_starts[g];
  }
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t len = prefix_lens[g];
    if (len < 0 || len % block_size != 0)
      return fail(PKV_ERR_INVALID,
                  "prefix_lens[%d] = %d must be a non-negative multiple of block_size %d", g,
                  len, block_size);
    if (len > max_context_len)
      return fail(PKV_ERR_INVALID, "prefix_lens[%d] = %d exceeds max_context_len %d", g, len,
                  max_context_len);
    out->prefix_len[g] = len;
  }
  return PKV_OK;
}

struct PrefixGeometry {
  int32_t part = 0;        // suffix partition
  int32_t split_keys = 0;  // keys per prefix split, a multiple of 64
  int32_t max_splits = 0;  // splits of the longest prefix (slots before the suffix's)
  int32_t slots = 0;       // partial slots per (row, head)
};

// Every prefix is split into key ranges of split_keys keys, the same for
// all groups (so the prefix launch's workgroups carry similar work), long
// enough that the launch has about a workgroup per CU (256) or more.  A
// row's slots: its group's prefix splits, then (from max_splits on) its
// suffix partitions.
int32_t prefix_geometry(int32_t num_heads, int32_t num_kv_heads, int32_t block_size,
                        int32_t max_context_len, const PrefixGroups& grp,
                        int32_t partition_size, PrefixGeometry* geo) {
  if (!is_pow2(block_size) || block_size < 16 || block_size > 256)
    return fail(PKV_ERR_UNSUPPORTED, "block_size must be a power of two in [16, 256]");
  int32_t min_prefix = max_context_len, max_prefix = 0;
  int64_t tiles = 0;  // row tiles of groups with a prefix
  for (int32_t g = 0; g < grp.count; ++g) {
    const int32_t rows = grp.start[g + 1] - grp.start[g];
    if (rows == 0) continue;
    min_prefix = std::min(min_prefix, grp.prefix_len[g]);
    max_prefix = std::max(max_prefix, grp.prefix_len[g]);
    if (grp.prefix_len[g] > 0) tiles += (rows + kPrefillRowsPerGroup - 1) / kPrefillRowsPerGroup;
  }
  const int32_t num_seqs = grp.start[grp.count];
  const int32_t suffix = max_context_len - std::min(min_prefix, max_prefix);
  int32_t st = resolve_partition(partition_size, block_size, num_seqs, num_kv_heads,
                                 std::max(1, suffix), &geo->part);
  if (st != PKV_OK) return st;
  if (max_prefix == 0) {
    geo->split_keys = 64;
    geo->max_splits = 0;
  } else {
    const int64_t pairs = int64_t(num_heads) * tiles;
    const int32_t key_tiles = (max_prefix + 63) / 64;
    const int32_t want = int32_t(std::min<int64_t>(key_tiles, std::max<int64_t>(1, (256 + pairs - 1) / pairs)));
    geo->split_keys = ((key_tiles + want - 1) / want) * 64;
    geo->max_splits = (max_prefix + geo->split_keys - 1) / geo->split_keys;
  }
  geo->slots = std::max(1, geo->max_splits + (suffix + geo->part - 1) / geo->part);
  if (geo->slots > 65535) return fail(PKV_ERR_UNSUPPORTED, "context too long");
  return PKV_OK;
}

// Workspace: [row records: num_seqs * 4 int32][acc: num_seqs * Hq * slots *
// D floats][(m, l): num_seqs * Hq * slots * 2 floats].
size_t prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                              int32_t slots) {
  return size_t(num_seqs) * 4 * sizeof(int32_t) +
         size_t(num_seqs) * num_heads * slots * (size_t(head_dim) + 2) * sizeof(float);
}

int32_t grouped_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_context_len,
                               int32_t num_groups, const int32_t* group_starts,
                               const int32_t* prefix_lens, int32_t partition_size,
                               size_t* bytes) {
  if (!bytes) return fail(PKV_ERR_INVALID, "NULL pointer argument");
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0)
    return fail(PKV_ERR_INVALID, "invalid sizes");
  PrefixGroups grp;
  int32_t st = read_groups(num_seqs, num_groups, group_starts, prefix_lens, block_size,
                           max_context_len, &grp);
  if (st != PKV_OK) return st;
  PrefixGeometry geo;
  st = prefix_geometry(num_heads, num_kv_heads, block_size, max_context_len, grp,
                       partition_size, &geo);
  if (st != PKV_OK) return st;
  *bytes = prefix_workspace_bytes(num_seqs, num_heads, head_dim, geo.slots);
  return ok();
}

// Lengths and groups of a step call checked against the sharing: the step
// stores each new row past its group's prefix and persists table changes
// from the suffix kernel, so a new row inside a prefix, or a change to a
// prefix entry or to a row with no suffix token, would break the sharing or
// never reach the device table.
int32_t check_step_against_groups(const PrefixGroups& grp, const int32_t* host_lens,
                                  bool new_rows, const int32_t* changes, int32_t num_changes,
                                  int32_t block_size, std::vector<int32_t>* row_prefix) {
  const int32_t num_seqs = grp.start[grp.count];
  row_prefix->assign(num_seqs, 0);
  for (int32_t g = 0; g < grp.count; ++g)
    for (int32_t r = grp.start[g]; r < grp.start[g + 1]; ++r) (*row_prefix)[r] = grp.prefix_len[g];
  if (num_seqs > 0 && !host_lens) return fail(PKV_ERR_INVALID, "context_lens is NULL");
  if (num_changes > 0 && !changes) return fail(PKV_ERR_INVALID, "changes is NULL");
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t pre = (*row_prefix)[i];
    if (new_rows && pre > 0 && host_lens[i] <= pre)
      return fail(PKV_ERR_INVALID,
                  "sequence %d: length %d leaves no suffix position for its new row", i,
                  host_lens[i]);
  }
  for (int32_t i = 0; i < num_changes; ++i) {
    const int32_t row = changes[3 * i], blk = changes[3 * i + 1];
    if (row < 0 || row >= num_seqs) continue;  // the step plan reports it
    const int32_t pre = (*row_prefix)[row];
    if (pre > 0 && (int64_t(blk) * block_size < pre || host_lens[row] <= pre))
      return fail(PKV_ERR_INVALID,
                  "table change %d (row %d, index %d) touches a shared prefix", i, row, blk);
  }
  return PKV_OK;
}

// The shared-prefix decode, with the lengths from the device (step == null)
// or by value with this step's table changes and new K/V rows (step form).
int32_t shared_prefix_call(const void* query, const void* key_new, const void* value_new,
                           const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t num_blocks, int32_t max_context_len, const PrefixGroups& grp,
                           float scale, int32_t partition_size, float* out, void* workspace,
                           size_t workspace_bytes_given, int32_t dtype, void* stream,
                           const StepPlan* step) {
  const bool shared_blocks = (dtype & PKV_DECODE_SHARED_BLOCKS) != 0;
  dtype &= ~int32_t(PKV_DECODE_SHARED_BLOCKS);
  if (dtype != PKV_BF16 && dtype != PKV_F16) {
    if (dtype_bytes(dtype) == 0) return fail(PKV_ERR_INVALID, "unknown dtype %d", dtype);
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode needs a float16 or bfloat16 cache");
  }
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_heads %d must be a positive multiple of num_kv_heads %d",
                num_heads, num_kv_heads);
  const int32_t G = num_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PKV_ERR_UNSUPPORTED, "heads per kv head must be 1, 2, 4 or 8 (got %d)", G);
  if (head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode supports head_dim 128 (got %d)",
                head_dim);
  if (max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID, "invalid table/pool sizes");
  if (int64_t(num_blocks) * block_size >= (int64_t(1) << 31))
    return fail(PKV_ERR_INVALID, "num_blocks * block_size must be below 2^31");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "scale must be finite");
  PrefixGeometry geo;
  int32_t st = prefix_geometry(num_heads, num_kv_heads, block_size, max_context_len, grp,
                               partition_size, &geo);
  if (st != PKV_OK) return st;
  for (int32_t g = 0; g < grp.count; ++g)
    if (int64_t(grp.prefix_len[g]) > int64_t(max_blocks_per_seq) * block_size)
      return fail(PKV_ERR_INVALID, "prefix_lens[%d] = %d exceeds the block table's capacity", g,
                  grp.prefix_len[g]);
  if (num_seqs == 0) return ok();
  if (!query || !key_cache || !value_cache || !block_tables || (!step && !context_lens) || !out)
    return fail(PKV_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) || !aligned16(out))
    return fail(PKV_ERR_INVALID, "query, caches and out must be 16-byte aligned");
  if (key_new || value_new) {
    if (!key_new || !value_new) return fail(PKV_ERR_INVALID, "key and value must both be given");
    if (!aligned16(key_new) || !aligned16(value_new))
      return fail(PKV_ERR_INVALID, "key and value must be 16-byte aligned");
  }
  const size_t need = prefix_workspace_bytes(num_seqs, num_heads, head_dim, geo.slots);
  if (!workspace || workspace_bytes_given < need)
    return fail(PKV_ERR_BUFFER_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes_given : size_t(0));
  if (!aligned16(workspace)) return fail(PKV_ERR_INVALID, "workspace must be 16-byte aligned");
  int32_t* row_info = static_cast<int32_t*>(workspace);
  float* ws_acc = reinterpret_cast<float*>(row_info + size_t(num_seqs) * 4);
  float* ws_ml = ws_acc + size_t(num_seqs) * num_heads * geo.slots * head_dim;

  // 1. every query against its group's prefix, on the matrix cores (also
  // every row's record: prefix length, the group's first row, prefix slots)
  hipError_t e = static_cast<hipError_t>(launch_prefix_partials(
      dtype, query, key_cache, value_cache, block_tables, grp, num_heads, num_kv_heads,
      block_size, max_blocks_per_seq, num_blocks, geo.split_keys, geo.max_splits, scale, ws_acc,
      ws_ml, row_info, geo.slots, stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefix launch: %s", hipGetErrorString(e));

  // 2. each sequence's private suffix, split-K, partials after the prefix's
  DecodeParams prm{};
  prm.query = static_cast<const uint8_t*>(query);
  prm.key_cache = static_cast<const uint8_t*>(key_cache);
  prm.value_cache = static_cast<const uint8_t*>(value_cache);
  prm.block_tables = block_tables;
  prm.block_tables_rw = const_cast<int32_t*>(block_tables);
  prm.context_lens = context_lens;
  prm.key_new = static_cast<const uint8_t*>(key_new);
  prm.value_new = static_cast<const uint8_t*>(value_new);
  prm.out = out;
  prm.ws_acc = ws_acc;
  prm.ws_ml = ws_ml;
  prm.num_kv_heads = num_kv_heads;
  while ((1 << prm.log2_bs) < block_size) ++prm.log2_bs;
  prm.max_blocks = max_blocks_per_seq;
  prm.num_blocks = num_blocks;
  prm.max_ctx = max_context_len;
  prm.part = geo.part;
  prm.max_parts = geo.slots;                                // workspace slots per row
  prm.grid_parts = std::max(1, geo.slots - geo.max_splits);  // suffix partitions
  prm.scale_log2 = scale * kLog2e;
  prm.v_scale = 1.0f;
  prm.shared_blocks = shared_blocks ? 1 : 0;
  prm.row_info = row_info;
  prm.slot_base = geo.max_splits;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (step) {
    for (size_t c = 0; c < step->chunks.size() && e == hipSuccess; ++c)
      e = dispatch_decode(dtype, head_dim, G, prm, step->chunks[c], step->ranks(c), s);
  } else {
    e = dispatch_decode(dtype, head_dim, G, prm, DeviceMeta{}, num_seqs, s);
  }
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(e));

  // 3. log-sum-exp merge of the prefix and suffix partials (every row)
  if (step) {
    for (size_t c = 0; c < step->chunks.size() && e == hipSuccess; ++c)
      e = launch_merge(prm, step->chunks[c], step->ranks(c), num_heads, head_dim, s);
  } else {
    e = launch_merge(prm, DeviceMeta{}, num_seqs, num_heads, head_dim, s);
  }
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode merge launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t grouped_call(const void* query, const void* key, const void* value,
                     const void* key_cache, const void* value_cache, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* changes, int32_t num_changes,
                     int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                     int32_t max_context_len, int32_t num_groups, const int32_t* group_starts,
                     const int32_t* prefix_lens, float scale, int32_t partition_size,
                     float* out, void* workspace, size_t workspace_bytes_given, int32_t dtype,
                     void* stream, bool step_form) {
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "negative num_seqs");
  if (num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "at most 65535 sequences per call");
  if (!is_pow2(block_size) || block_size < 16 || block_size > 256)
    return fail(PKV_ERR_UNSUPPORTED, "block_size must be a power of two in [16, 256]");
  if (max_context_len < 0) return fail(PKV_ERR_INVALID, "negative max_context_len");
  PrefixGroups grp;
  int32_t st = read_groups(num_seqs, num_groups, group_starts, prefix_lens, block_size,
                           max_context_len, &grp);
  if (st != PKV_OK) return st;
  if (!step_form)
    return shared_prefix_call(query, nullptr, nullptr, key_cache, value_cache, block_tables,
                              context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                              block_size, max_blocks_per_seq, num_blocks, max_context_len, grp,
                              scale, partition_size, out, workspace, workspace_bytes_given, dtype,
                              stream, nullptr);
  if (num_changes < 0) return fail(PKV_ERR_INVALID, "negative num_changes");
  std::vector<int32_t> row_prefix;
  st = check_step_against_groups(grp, context_lens, key != nullptr, changes, num_changes,
                                 block_size, &row_prefix);
  if (st != PKV_OK) return st;
  StepPlan plan;
  st = make_step_plan(context_lens, changes, num_changes, num_seqs, num_kv_heads,
                      max_blocks_per_seq, &plan, row_prefix.data());
  if (st != PKV_OK) return st;
  return shared_prefix_call(query, key, value, key_cache, value_cache, block_tables, nullptr,
                            num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, num_blocks, max_context_len, grp, scale,
                            partition_size, out, workspace, workspace_bytes_given, dtype, stream,
                            &plan);
}
}  // namespace

extern "C" int32_t pkv_paged_attention_decode_shared_prefix_workspace_size(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_context_len, int32_t prefix_len, int32_t partition_size,
    size_t* bytes) {
  if (prefix_len <= 0)
    return fail(PKV_ERR_INVALID, "prefix_len %d must be a positive multiple of block_size %d",
                prefix_len, block_size);
  const int32_t starts[2] = {0, num_seqs};
  return grouped_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                max_context_len, 1, starts, &prefix_len, partition_size, bytes);
}

extern "C" int32_t pkv_paged_attention_decode_shared_prefix(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
    int32_t prefix_len, float scale, int32_t partition_size, float* out, void* workspace,
    size_t workspace_bytes_given, int32_t dtype, void* stream) {
  if (prefix_len <= 0)
    return fail(PKV_ERR_INVALID, "prefix_len %d must be a positive multiple of block_size %d",
                prefix_len, block_size);
  const int32_t starts[2] = {0, std::max(num_seqs, 0)};
  return grouped_call(query, nullptr, nullptr, key_cache, value_cache, block_tables,
                      context_lens, nullptr, 0, num_seqs, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, max_context_len, 1, starts,
                      &prefix_len, scale, partition_size, out, workspace, workspace_bytes_given,
                      dtype, stream, false);
}

extern "C" int32_t pkv_paged_attention_decode_shared_prefix_step(
    const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, int32_t* block_tables, const int32_t* context_lens,
    const int32_t* changes, int32_t num_changes, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t num_blocks, int32_t max_context_len, int32_t prefix_len, float scale,
    int32_t partition_size, float* out, void* workspace, size_t workspace_bytes_given,
    int32_t dtype, void* stream) {
  if (prefix_len <= 0)
    return fail(PKV_ERR_INVALID, "prefix_len %d must be a positive multiple of block_size %d",
                prefix_len, block_size);
  const int32_t starts[2] = {0, std::max(num_seqs, 0)};
  return grouped_call(query, key, value, key_cache, value_cache, block_tables, context_lens,
                      changes, num_changes, num_seqs, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, max_context_len, 1, starts,
                      &prefix_len, scale, partition_size, out, workspace, workspace_bytes_given,
                      dtype, stream, true);
}

extern "C" int32_t pkv_paged_attention_decode_grouped_prefix_workspace_size(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_context_len, int32_t num_groups,
    const int32_t* group_starts, const int32_t* prefix_lens, int32_t partition_size,
    size_t* bytes) {
  return grouped_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                max_context_len, num_groups, group_starts, prefix_lens,
                                partition_size, bytes);
}

extern "C" int32_t pkv_paged_attention_decode_grouped_prefix(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
    int32_t num_groups, const int32_t* group_starts, const int32_t* prefix_lens, float scale,
    int32_t partition_size, float* out, void* workspace, size_t workspace_bytes_given,
    int32_t dtype, void* stream) {
  return grouped_call(query, nullptr, nullptr, key_cache, value_cache, block_tables,
                      context_lens, nullptr, 0, num_seqs, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, max_context_len, num_groups,
                      group_starts, prefix_lens, scale, partition_size, out, workspace,
                      workspace_bytes_given, dtype, stream, false);
}

extern "C" int32_t pkv_paged_attention_decode_grouped_prefix_step(
    const void* query, const void* key, const void* value, void* key_cache,
    void* value_cache, int32_t* block_tables, const int32_t* context_lens,
    const int32_t* changes, int32_t num_changes, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t num_blocks, int32_t max_context_len, int32_t num_groups,
    const int32_t* group_starts, const int32_t* prefix_lens, float scale,
    int32_t partition_size, float* out, void* workspace, size_t workspace_bytes_given,
    int32_t dtype, void* stream) {
  return grouped_call(query, key, value, key_cache, value_cache, block_tables, context_lens,
                      changes, num_changes, num_seqs, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, max_context_len, num_groups,
                      group_starts, prefix_lens, scale, partition_size, out, workspace,
                      workspace_bytes_given, dtype, stream, true);
}

// ---- decode with no allocation at all: split-K partials in a fixed array --

namespace {
// The split-K partials of pkv_paged_attention_decode_noalloc.  Every GPU
// the library runs on holds its own copy from the time the library's code
// is loaded there until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// device copy): the device address comes from hipGetSymbolAddress, per
// device, below.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device `stream` runs on, looked
// up once per device with that device current.
int32_t scratch_for_stream(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "stream device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, "device %d beyond the %d this library serves", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int current = 0;
    e = hipGetDevice(&current);
    if (e == hipSuccess && current != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (current != dev) {
      const hipError_t back = hipSetDevice(current);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess || !p)
      return fail(PKV_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}
}  // namespace

extern "C" int32_t pkv_paged_attention_decode_noalloc(
    const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, float* out, int32_t dtype, void* stream) {
  size_t need = 0;
  int32_t st = pkv_paged_attention_decode_workspace_size(
      num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size, &need);
  if (st != PKV_OK) return st;
  if (need > kScratchBytes)
    return fail(PKV_ERR_BUFFER_TOO_SMALL,
                "these sizes need %zu bytes of split-K partials, beyond the %zu bytes of the "
                "library's fixed scratch array (use pkv_paged_attention_decode with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_for_stream(static_cast<hipStream_t>(stream), &ws);
    if (st != PKV_OK) return st;
  }
  return run_decode(query, nullptr, nullptr, key_cache, value_cache, block_tables, context_lens,
                    num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                    num_blocks, max_context_len, scale, partition_size, out, ws,
                    need > 0 ? kScratchBytes : 0, dtype, stream, true, true, nullptr);
}
