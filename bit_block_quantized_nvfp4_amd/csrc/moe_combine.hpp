// The combine of one token and 8 consecutive columns (A10):
//   out[t][c..c+8) = bf16( sum_k w[t][k] * y[slot_pos[t*K+k]] + g_t * y[slot_pos[T*K+t]] )
// g_t = 1, or sigmoid(gate[t]) for a gated shared expert; fp32 accumulation in
// slot order, then the shared expert, one rounding at the end (the same-order
// rule for per-slot expert outputs of the issue "EXL3 Qwen3.8-Flash-Next on
// CUDA sm_120 ...", expert-parallel TP=2).  combine_rows reads the 8 values
// of slot position p at yrow(p): the combine kernel reads y in global memory,
// the decode down + combine kernel its LDS copy of the same values, so both
// give the same bits.
#pragma once

#include <math.h>

#include "moe_device.hpp"

namespace moe {

template <typename YRow>
__device__ __forceinline__ void combine_rows(YRow yrow, const float* __restrict__ w,
                                             const int32_t* __restrict__ slot_pos,
                                             const float* __restrict__ gate, int T, int K,
                                             int has_shared, uint16_t* __restrict__ dst, int t) {
  const int TK = T * K;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const int ps = has_shared ? slot_pos[(size_t)TK + t] : -1;
  // slots in batches of 16: all positions and weights of a batch are loaded,
  // then all of its rows, then accumulated in slot order
  for (int k0 = 0; k0 < K; k0 += 16) {
    int p[16];
    float wt[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int k = k0 + j;
      p[j] = (k < K) ? slot_pos[(size_t)t * K + k] : -1;
      wt[j] = (k < K) ? w[(size_t)t * K + k] : 0.f;
    }
    u32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      v[j] = (p[j] >= 0 && p[j] < TK) ? *(const u32x4*)yrow(p[j]) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (p[j] >= 0 && p[j] < TK) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(wt[j], bf16_bits_to_f32(v[j][q] & 0xFFFFu), acc[2 * q]);
          acc[2 * q + 1] = fmaf(wt[j], bf16_bits_to_f32(v[j][q] >> 16), acc[2 * q + 1]);
        }
      }
    }
  }
  if (ps >= 0 && ps < TK + T) {
    const u32x4 v = *(const u32x4*)yrow(ps);
    if (gate) {  // sigmoid-gated shared expert
      const float sg = 1.0f / (1.0f + expf(-gate[t]));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = fmaf(sg, bf16_bits_to_f32(v[j] & 0xFFFFu), acc[2 * j]);
        acc[2 * j + 1] = fmaf(sg, bf16_bits_to_f32(v[j] >> 16), acc[2 * j + 1]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += bf16_bits_to_f32(v[j] & 0xFFFFu);
        acc[2 * j + 1] += bf16_bits_to_f32(v[j] >> 16);
      }
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
  *(u32x4*)dst = o;
}

// Columns [col, col + 8) of token t, with y [S][H] in global memory.
__device__ __forceinline__ void combine_chunk(const uint16_t* __restrict__ y,
                                              const float* __restrict__ w,
                                              const int32_t* __restrict__ slot_pos,
                                              const float* __restrict__ gate, int T, int K, int H,
                                              int has_shared, uint16_t* __restrict__ out, int t,
                                              int col) {
  combine_rows([&](int p) { return y + (size_t)p * H + col; }, w, slot_pos, gate, T, K, has_shared,
               out + (size_t)t * H + col, t);
}

}  // namespace moe
