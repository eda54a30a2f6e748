// Device helpers shared by the gfx950 kernels: score keys, bf16 packing,
// wavefront (64-lane) and workgroup reductions/scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvpop_internal.h"

namespace kvpop {

constexpr int WAVE = 64;

// Raw buffer descriptor, last word: 32-bit data format (untyped access).
// Loads past the descriptor's byte count return 0 without a memory access.
constexpr int BUF_RSRC_WORD3 = 0x00020000;

// Order-preserving code of a float32 score: flipping all bits of negatives
// and setting the sign bit of non-negatives makes unsigned order equal float
// order.  -0 is folded onto +0 first so the two compare equal.
__device__ __forceinline__ uint32_t score_code(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score of an order code (the inverse of score_code; -0 comes back as +0).
__device__ __forceinline__ float code_value(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ bool score_is_nan(float s) {
  return (__float_as_uint(s) & 0x7FFFFFFFu) > 0x7F800000u;
}

__device__ __forceinline__ uint64_t make_key(uint32_t code, int32_t pos) {
  return (static_cast<uint64_t>(code) << 32) | static_cast<uint32_t>(pos);
}

// bf16 pair packed in a 32-bit word -> two floats (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---- wavefront reductions --------------------------------------------------

// Inclusive prefix sum over the 64 lanes with DPP: shifts by 1, 2, 4 and 8
// lanes within each row of 16, then the row broadcasts of lane 15 (into rows
// 1 and 3) and lane 31 (into rows 2 and 3).  Lanes without a source add the
// `old` operand, 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_add_src(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_inclusive_scan_u32(uint32_t x) {
  x += dpp_add_src<0x111, 0xF>(x);  // row_shr:1
  x += dpp_add_src<0x112, 0xF>(x);  // row_shr:2
  x += dpp_add_src<0x114, 0xF>(x);  // row_shr:4
  x += dpp_add_src<0x118, 0xF>(x);  // row_shr:8
  x += dpp_add_src<0x142, 0xA>(x);  // row_bcast:15
  x += dpp_add_src<0x143, 0xC>(x);  // row_bcast:31
  return x;
}

// Lexicographic minimum of (key, slot) over the wavefront.
__device__ __forceinline__ void wave_min_key(uint64_t& key, int32_t& slot) {
#pragma unroll
  for (int d = WAVE / 2; d >= 1; d >>= 1) {
    uint64_t k2 = __shfl_xor(key, d, WAVE);
    int32_t s2 = __shfl_xor(slot, d, WAVE);
    if (k2 < key || (k2 == key && s2 < slot)) {
      key = k2;
      slot = s2;
    }
  }
}

// Exclusive scan of one u32 per thread over a workgroup of NT threads.
// `scratch` must hold NT/64 + 1 words of LDS.  Returns the exclusive prefix;
// *total receives the sum over the workgroup.  Must be called by all threads.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan_u32(uint32_t x, uint32_t* scratch,
                                                             uint32_t* total) {
  constexpr int NW = NT / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = threadIdx.x / WAVE;
  uint32_t inc = wave_inclusive_scan_u32(x);
  if (lane == WAVE - 1) scratch[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    uint32_t w = lane < NW ? scratch[lane] : 0u;
    uint32_t wi = wave_inclusive_scan_u32(w);
    if (lane < NW) scratch[lane] = wi - w;  // exclusive over waves
    if (lane == NW - 1) scratch[NW] = wi;
  }
  __syncthreads();
  uint32_t ex = scratch[wid] + inc - x;
  *total = scratch[NW];
  __syncthreads();  // scratch may be reused right after
  return ex;
}

}  // namespace kvpop
