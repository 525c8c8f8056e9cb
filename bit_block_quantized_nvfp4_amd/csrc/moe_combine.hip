// Combine (A10): out[t] = bf16( sum_k w[t][k] * y[slot_pos[t*K+k]] + c_t y[slot_pos[T*K+t]] ),
// c_t = 1, or sigmoid(gate[t]) for the gated shared expert (combine_chunk in
// moe_combine.hpp).  Each thread owns 8 consecutive columns of one token
// (16-byte loads/stores); the order of the sum is fixed per element and
// independent of how the grid is cut.
#include "moe_combine.hpp"
#include "moe_internal.hpp"

namespace moe {

__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y,
                                                 const float* __restrict__ w,
                                                 const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ gate, int T, int K,
                                                 int H, int has_shared,
                                                 uint16_t* __restrict__ out) {
  const int cpr = H / 8;  // 8-column chunks per row
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long)T * cpr) return;
  const int t = (int)(gid / cpr), c = (int)(gid % cpr);
  combine_chunk(y, w, slot_pos, gate, T, K, H, has_shared, out, t, 8 * c);
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
