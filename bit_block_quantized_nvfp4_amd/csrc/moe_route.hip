// Router top-K + softmax over the selected logits (A1).
//
// One wave64 per token.  Lane l holds logits l, l+64, l+128, ... in registers
// (coalesced 256-byte loads).  K rounds of a wave arg-max pick the experts in
// rank order; the arg-max key is (logit descending, index ascending), NaN is
// read as -inf, which is the tie rule of the page "handover briefs" (item A1
// and the indexer-selection kernel spec: rank(b) counts the j with s_j > s_b or
// s_j == s_b and j < b).  The weights are the softmax of the K selected logits
// (equal to the renormalised full softmax), computed in fp32 with a fixed-order
// butterfly sum.
#include <limits.h>
#include <math.h>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

template <int MAXV>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T,
                                                     int E, int K, int32_t* __restrict__ ids,
                                                     float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + (size_t)t * E;

  float v[MAXV];
  uint32_t absent = 0;  // bit j: element j is selected already or does not exist
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int e = lane + 64 * j;
    float z = -INFINITY;
    if (e < E) z = row[e];
    else absent |= 1u << j;
    v[j] = (z != z) ? -INFINITY : z;
  }

  float zsel = -INFINITY;
  int isel = 0;
  for (int k = 0; k < K; ++k) {
    // best untaken element of this lane: indices ascend with j, so a strict '>'
    // keeps the lower index among equal values
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
      const bool free_j = !((absent >> j) & 1u);
      if (free_j && (bi == INT_MAX || v[j] > bv)) {
        bv = v[j];
        bi = lane + 64 * j;
      }
    }
    // wave arg-max under (value desc, index asc); a total order, so the
    // butterfly leaves the same winner in every lane
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == k) {
      zsel = bv;
      isel = bi;
    }
    if ((bi & 63) == lane) absent |= 1u << (bi >> 6);  // bi < E because K <= E
  }

  const float z0 = __shfl(zsel, 0, 64);
  float ex = 0.f;
  if (lane < K) ex = expf(zsel == z0 ? 0.f : zsel - z0);
  const float sum = wave_sum(ex);
  if (lane < K) {
    ids[(size_t)t * K + lane] = isel;
    w[(size_t)t * K + lane] = ex / sum;
  }
}

void register_route_kernels(std::vector<const void*>& k) {
  k.push_back((const void*)&k_route_topk<1>);
  k.push_back((const void*)&k_route_topk<2>);
  k.push_back((const void*)&k_route_topk<4>);
  k.push_back((const void*)&k_route_topk<8>);
  k.push_back((const void*)&k_route_topk<16>);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                             hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64) MOE_LAUNCH("route_topk", s, (k_route_topk<1>), grid, block, 0, s, logits, T, E, K, ids, w);
  else if (E <= 128) MOE_LAUNCH("route_topk", s, (k_route_topk<2>), grid, block, 0, s, logits, T, E, K, ids, w);
  else if (E <= 256) MOE_LAUNCH("route_topk", s, (k_route_topk<4>), grid, block, 0, s, logits, T, E, K, ids, w);
  else if (E <= 512) MOE_LAUNCH("route_topk", s, (k_route_topk<8>), grid, block, 0, s, logits, T, E, K, ids, w);
  else MOE_LAUNCH("route_topk", s, (k_route_topk<16>), grid, block, 0, s, logits, T, E, K, ids, w);
  return hipGetLastError();
}

}  // namespace moe
