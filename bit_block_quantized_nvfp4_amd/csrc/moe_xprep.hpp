// Activation-row prep of the grouped path, one 256-thread block per token
// row (H <= 4096): the row's absmax, then
//   bf16 arm: f16 row x * 2^sh with sh bringing the absmax into [2^14, 2^15)
//             (exact for every value above 2^-29 of the absmax), unmul = 2^-sh;
//   FP8 arm:  the row quantisation s = absmax / 448, codes e4m3(x / s) (to xq,
//             s to xs), and the exact f16 value of each code, unmul = s.
// The products with the NVFP4 weights then run on f16 MFMA and the epilogue
// multiplies the f32 sums by unmul.
#pragma once

#include <math.h>

#include "moe_device.hpp"
#include "moe_ffn_common.hpp"

namespace moe {

// Row t; every thread of the block calls it (one barrier inside); wmax is a
// 4-float LDS array of the block.
template <bool FP8>
__device__ __forceinline__ void xprep_row(const uint16_t* __restrict__ x, int H, int t,
                                          _Float16* __restrict__ xh, float* __restrict__ unmul,
                                          uint8_t* __restrict__ xq, float* __restrict__ xs,
                                          float* wmax) {
  const int tid = threadIdx.x;
  const u32x4* row = (const u32x4*)(x + (size_t)t * H);
  u32x4 v[2];
  float amax = 0.f;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int c = tid + 256 * cc;
    if (c < H / 8) {
      v[cc] = row[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[cc][j] & 0xFFFFu)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[cc][j] >> 16)));
      }
    }
  }
  amax = wave_max_nonneg(amax);  // fmaxf drops NaN: every lane is >= 0, not NaN
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float mul;
  if (FP8) {
    // the row quantisation of the FP8 arm: s = absmax/448, codes e4m3(x * 448/absmax)
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    mul = amax > 0.f ? 448.0f / amax : 1.0f;
    if (tid == 0) {
      xs[t] = s;
      unmul[t] = s;
    }
  } else {
    const int sh = f16_row_shift(amax);
    mul = ldexpf(1.0f, sh);
    if (tid == 0) unmul[t] = ldexpf(1.0f, -sh);
  }
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int c = tid + 256 * cc;
    if (c < H / 8) {
      u32x4 o;
      if (FP8) {
        u32x2 code;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float f0 = bf16_bits_to_f32(v[cc][2 * j] & 0xFFFFu) * mul;
          float f1 = bf16_bits_to_f32(v[cc][2 * j] >> 16) * mul;
          float f2 = bf16_bits_to_f32(v[cc][2 * j + 1] & 0xFFFFu) * mul;
          float f3 = bf16_bits_to_f32(v[cc][2 * j + 1] >> 16) * mul;
          f0 = fminf(fmaxf(f0, -448.f), 448.f);
          f1 = fminf(fmaxf(f1, -448.f), 448.f);
          f2 = fminf(fmaxf(f2, -448.f), 448.f);
          f3 = fminf(fmaxf(f3, -448.f), 448.f);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, w, true);
          code[j] = (uint32_t)w;
        }
        *(u32x2*)(xq + (size_t)t * H + 8 * c) = code;
        const u32x2 lo = fp8x4_to_f16(code.x), hi = fp8x4_to_f16(code.y);
        o = u32x4{lo.x, lo.y, hi.x, hi.y};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = pack_f16x2(bf16_bits_to_f32(v[cc][j] & 0xFFFFu) * mul,
                            bf16_bits_to_f32(v[cc][j] >> 16) * mul);
      }
      *(u32x4*)(xh + (size_t)t * H + 8 * c) = o;
    }
  }
}

}  // namespace moe
