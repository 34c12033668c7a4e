// Device-side helpers shared by the gfx950 kernels: vector types, bf16 packing,
// wave reductions and launch error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace vmoba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 of two values, packed lo | hi << 16 (one
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// acc + lo + hi of a packed bf16 pair, in fp32 (one v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// NaN-propagating maximum of three values (one v_maximum3_f32).  Unlike fmaxf it needs no
// canonicalisation of operands that come straight from the matrix cores.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// x from the lane that DPP control CTRL names (a permutation inside each row of 16).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(x)), CTRL, 0xf, 0xf, false));
  const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(x >> 32)), CTRL, 0xf, 0xf, false));
  return (uint64_t(hi) << 32) | lo;
}

// Sum over the 64 lanes of a wave, returned to every lane, without going through LDS:
// DPP swaps inside quads (lane ^ 1, ^ 2), then mirrors inside half rows and rows of 16,
// then the swaps of rows 0/1 with 2/3... (lane ^ 16) and of the two halves (lane ^ 32).
// Precondition: all 64 lanes are active.  The DPP moves (bound_ctrl off) and the permlane
// swaps read the registers of inactive lanes as they stand, so a call from divergent code
// would add stale values.  Builds with VMOBA_DEVICE_CHECKS trap on a partial wave.
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#ifdef VMOBA_DEVICE_CHECKS
  if (__builtin_amdgcn_read_exec() != ~0ull) __builtin_trap();
#endif
  v += dpp_u64<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_u64<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_u64<0x141>(v);   // row_half_mirror
  v += dpp_u64<0x140>(v);   // row_mirror
  const uint32_t lo = uint32_t(v), hi = uint32_t(v >> 32);
  const auto l16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  v = ((uint64_t(h16[0]) << 32) | l16[0]) + ((uint64_t(h16[1]) << 32) | l16[1]);
  const uint32_t lo2 = uint32_t(v), hi2 = uint32_t(v >> 32);
  const auto l32 = __builtin_amdgcn_permlane32_swap(lo2, lo2, false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap(hi2, hi2, false, false);
  return ((uint64_t(h32[0]) << 32) | l32[0]) + ((uint64_t(h32[1]) << 32) | l32[1]);
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? VMOBA_OK : VMOBA_ERR_HIP;
}

}  // namespace vmoba
