// Device helpers shared by the expert-FFN kernels: NVFP4 -> MFMA operand
// conversion (bf16 and f16), e4m3 activation conversion, SiLU, slot -> token.
#pragma once

#include <math.h>

#include "moe_device.hpp"

namespace moe {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---- NVFP4 -> bf16 operand: v_cvt_scalef32_pk_f32_fp4 gives the two e2m1
// values of a byte (its scale operand carries only a power of two, so the
// e4m3 block scale is applied by an f32 multiply), v_cvt_pk_bf16_f32 packs
// them.  e2m1 x e4m3 has <= 6 significant bits: the bf16 value is exact.
template <int B>
__device__ __forceinline__ uint32_t dq_pair(uint32_t word, float s) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, B);
  v = v * s;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 8 e2m1 codes (one 32-bit word, element 2j in the low nibble of byte j)
// times their block scale -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 dq8(uint32_t word, float s) {
  u32x4 r = {dq_pair<0>(word, s), dq_pair<1>(word, s), dq_pair<2>(word, s), dq_pair<3>(word, s)};
  return __builtin_bit_cast(bf16x8, r);
}

// ---- NVFP4 -> f16 operand: v_cvt_scalef32_pk_f16_fp4 (two e2m1 values of a
// byte, exact in f16) and v_pk_mul_f16 by the block scale held as an f16
// (e4m3 fits f16 exactly; the product, <= 6 significant bits in
// [2^-10, 2688], is exact too).  One instruction per element.
template <int B>
__device__ __forceinline__ uint32_t dqh_pair(uint32_t word, _Float16 s) {
  f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, B);
  const f16x2 ss = {s, s};
  return __builtin_bit_cast(uint32_t, v * ss);
}

__device__ __forceinline__ f16x8 dqh8(uint32_t word, _Float16 s) {
  u32x4 r = {dqh_pair<0>(word, s), dqh_pair<1>(word, s), dqh_pair<2>(word, s),
             dqh_pair<3>(word, s)};
  return __builtin_bit_cast(f16x8, r);
}

// Two e4m3 scale bytes (low 16 bits of w) -> two f16 values.
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

// 8 e4m3 activation codes (two 32-bit words) -> one bf16x8 operand (exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  u32x4 r;
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.x, 1.0f, false);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.x, 1.0f, true);
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.y, 1.0f, false);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.y, 1.0f, true);
  r.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2));
  r.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2));
  r.z = __builtin_bit_cast(uint32_t, __builtin_convertvector(c, bf16x2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_convertvector(d, bf16x2));
  return __builtin_bit_cast(bf16x8, r);
}

// 4 e4m3 activation codes (one 32-bit word) -> two packed f16 pairs (exact).
__device__ __forceinline__ u32x2 fp8x4_to_f16(uint32_t w) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// One global -> LDS DMA of 16 bytes per lane: lane l's 16 bytes at g land at
// lds + 16*l (lds is wave-uniform).  Completion is tracked like a load
// (vmcnt); a barrier after the wait makes the data visible to the block.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// silu(g) = g * sigma(g), sigma(g) = 1 / (1 + exp(-g)), with the hardware
// v_exp_f32 (2^x) and v_rcp_f32 (each ~1 ulp in f32): the result is rounded
// to bf16 (2^-9 relative) right after, so correctly rounded exp and division
// would buy nothing.  Finite g far below zero gives -0 (exp2 overflows to
// +inf and rcp(+inf) = 0); g far above zero gives g.
__device__ __forceinline__ float silu_f32(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Token of a sorted slot: routed slot s -> s / K, shared slot T*K + t -> t,
// anything else -> -1 (the row is skipped).
__device__ __forceinline__ int slot_token(int sl, int T, int K, int has_shared) {
  const int TK = T * K;
  if (sl >= 0 && sl < TK) return sl / K;
  if (has_shared && sl >= TK && sl < TK + T) return sl - TK;
  return -1;
}

// Power-of-two shift that brings a row's absmax into [2^14, 2^15) so that the
// row fits f16 with headroom (f16 max 65504); bf16 values times 2^sh are then
// exact in f16 unless below 2^-14 after the shift (i.e. below ~2^-29 of the
// row's absmax).  Clamped to +-100 so both 2^sh and 2^-sh are normal f32.
__device__ __forceinline__ int f16_row_shift(float amax) {
  if (!(amax > 0.f) || !(amax < INFINITY)) return 0;
  int e;
  (void)frexpf(amax, &e);  // amax = m * 2^e, m in [0.5, 1)
  int sh = 15 - e;
  return sh > 100 ? 100 : (sh < -100 ? -100 : sh);
}

}  // namespace moe
