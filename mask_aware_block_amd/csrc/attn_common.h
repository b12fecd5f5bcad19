// Per-wave helpers shared by the bf16 MFMA attention kernels for gfx950
// (attn_bf16_o3.hip, attn_bf16_pair.hip): vector types, the LDS swizzles of
// K and V tiles, lane-pair reductions and the softmax constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"

namespace fmask {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS FMASK_LDS_AS
#define INLINE __attribute__((always_inline))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 4294967296.f;  // 2^kLazyLog2 with kLazyLog2 = 32: bound on a lane's share of a row sum
constexpr int kQkAhead = 3;  // K fragments read ahead of their MFMA
constexpr int kPvAhead = 3;  // V^T fragments read ahead of their MFMA

// Block info of a 64 x 64 bitmap block: its pool index if PARTIAL, else
// kBlkFull or kBlkSkip.
constexpr int kBlkFull = -1, kBlkSkip = -2;

// LDS swizzles of a K / V tile row (KCH 16-byte chunks per row): the chunk
// index is XORed with these so that MFMA operand reads are conflict-free.
template <int KCH>
__device__ inline int kswz(int key) { return key & (KCH - 1); }
template <int KCH>
__device__ inline int vswz(int key) {
  return KCH == 16 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
}

// max / sum of x over lanes l and l ^ 32.  v_permlane32_swap of x with itself
// leaves {x[l], x[l ^ 32]} in some order in the two results (no LDS round
// trip, unlike a lane shuffle).
__device__ inline float pair_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ inline float pair_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

}  // namespace
}  // namespace fmask
