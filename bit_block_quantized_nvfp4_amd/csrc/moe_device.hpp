// Device-side helpers shared by the gfx950 kernels of the NVFP4 MoE layer:
// vector types, bf16 <-> f32, wave-level reductions and scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even f32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 r = (__bf16)f;
  return __builtin_bit_cast(uint16_t, r);
}

// Two f32 -> packed bf16 pair (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

// ---- wave-level reductions and scans on DPP (no LDS round trips; every
// result is order-fixed and uniform or per lane as stated) ----

// DPP move of v from the lane that control CTRL names (all rows and banks).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
// The same, written only in the rows of mask ROWS (other lanes keep v).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_rows(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}
// Max over the 64 lanes, as a uniform value, without LDS: DPP xor-1, xor-2
// (quad permutes), half-row and row mirrors leave each row's max in all its
// lanes; row broadcasts of lane 15 (into rows 1, 3) and lane 31 (into rows
// 2, 3) leave the wave's max in lane 63.
// Each step moves with 0 (the identity of the max) in the lanes a row mask
// leaves out, which lets the compiler fold the move into the max (one DPP
// max per step).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto mv = [](uint32_t x, auto ctrl, auto rows) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value,
                                                 decltype(rows)::value, 0xF, false);
  };
  using RA = std::integral_constant<int, 0xF>;
  v = max(v, mv(v, std::integral_constant<int, 0xB1>{}, RA{}));
  v = max(v, mv(v, std::integral_constant<int, 0x4E>{}, RA{}));
  v = max(v, mv(v, std::integral_constant<int, 0x141>{}, RA{}));
  v = max(v, mv(v, std::integral_constant<int, 0x140>{}, RA{}));
  v = max(v, mv(v, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{}));
  v = max(v, mv(v, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{}));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Sum over the 64 lanes, as a uniform value, in a fixed order and without
// LDS: the same DPP steps as wave_max_u32 with adds.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  auto mv = [](float x, auto ctrl, auto rows) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                      decltype(rows)::value, 0xF, false));
  };
  using C1 = std::integral_constant<int, 0xB1>;
  using C2 = std::integral_constant<int, 0x4E>;
  using C3 = std::integral_constant<int, 0x141>;
  using C4 = std::integral_constant<int, 0x140>;
  using C5 = std::integral_constant<int, 0x142>;
  using C6 = std::integral_constant<int, 0x143>;
  using RA = std::integral_constant<int, 0xF>;
  v += mv(v, C1{}, RA{});
  v += mv(v, C2{}, RA{});
  v += mv(v, C3{}, RA{});
  v += mv(v, C4{}, RA{});
  v += mv(v, C5{}, std::integral_constant<int, 0xA>{});
  v += mv(v, C6{}, std::integral_constant<int, 0xC>{});
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Max over the lanes of a float that is >= 0 and not NaN in every lane (the
// bit patterns of such floats order like their values).
__device__ __forceinline__ float wave_max_nonneg(float v) {
  return __uint_as_float(wave_max_u32(__float_as_uint(v)));
}

// Inclusive prefix sum over the 64 lanes of a wave, without LDS: row shifts
// by 1, 2, 4, 8 (a lane with no source adds 0) give each row of 16 lanes its
// own prefix sums; row broadcasts of lane 15 (into rows 1, 3) and lane 31
// (into rows 2, 3) add the totals of the rows before.  lane is unused (kept
// for the callers' symmetry with the 64-bit scan).
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  (void)lane;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

}  // namespace moe
