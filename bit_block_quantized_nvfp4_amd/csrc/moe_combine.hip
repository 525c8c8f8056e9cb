// Combine (A10): out[t] = bf16( sum_k w[t][k] * y[slot_pos[t*K+k]] + c_t y[slot_pos[T*K+t]] ),
// c_t = 1, or sigmoid(gate[t]) for the gated shared expert; fp32 accumulation in slot order then the shared expert, one rounding at the
// end.  The order is fixed per element and independent of how the grid is cut
// (the same-order rule for per-slot expert outputs of the issue "EXL3
// Qwen3.8-Flash-Next on CUDA sm_120 ...", expert-parallel TP=2).
// Each thread owns 8 consecutive columns of one token (16-byte loads/stores).
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y,
                                                 const float* __restrict__ w,
                                                 const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ gate, int T,
                                                 int K, int H, int has_shared,
                                                 uint16_t* __restrict__ out) {
  const int cpr = H / 8;  // 8-column chunks per row
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long)T * cpr) return;
  const int t = (int)(gid / cpr), c = (int)(gid % cpr);
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
      v[j] = (p[j] >= 0 && p[j] < TK) ? *(const u32x4*)(y + (size_t)p[j] * H + 8 * c) : u32x4{0u, 0u, 0u, 0u};
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
    const u32x4 v = *(const u32x4*)(y + (size_t)ps * H + 8 * c);
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
  *(u32x4*)(out + (size_t)t * H + 8 * c) = o;
}

void register_combine_kernels(std::vector<const void*>& k) { k.push_back((const void*)&k_combine); }

hipError_t launch_combine(const uint16_t* y, const float* w, const int32_t* slot_pos,
                          const float* gate, int T, int K, int H, int has_shared, uint16_t* out,
                          hipStream_t s) {
  const long n = (long)T * (H / 8);
  MOE_LAUNCH("combine", s, k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y, w,
             slot_pos, gate, T, K, H, has_shared, out);
  return hipGetLastError();
}

}  // namespace moe
