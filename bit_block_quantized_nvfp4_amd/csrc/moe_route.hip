// Router top-K + softmax over the selected logits (A1).
//
// One wave64 per token.  Lane l holds logits l, l+64, l+128, ... in registers
// (coalesced 256-byte loads) and sorts its own keys once, largest first (a
// stable odd-even transposition sort, so equal keys stay in index order).
// Each of the K rounds then takes one wave max over the 64 list heads (DPP
// inside rows of 16 lanes, row broadcasts across rows); the lane holding it
// pops its head.  When several heads hold the max, the lowest expert index
// wins (a wave min over those heads).  The arg-max key is (logit descending,
// index ascending), NaN is read as -inf, which is the tie rule of the page
// "handover briefs" (item A1 and the indexer-selection kernel spec: rank(b)
// counts the j with s_j > s_b or s_j == s_b and j < b).  The weights are the
// softmax of the K selected logits (equal to the renormalised full softmax),
// computed in fp32 with a fixed-order DPP sum.
#include "moe_internal.hpp"
#include "moe_topk.hpp"

namespace moe {

template <int MAXV>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T,
                                                     int E, int K, int32_t* __restrict__ ids,
                                                     float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  route_row_topk<MAXV>(logits + (size_t)t * E, E, K, ids + (size_t)t * K, w + (size_t)t * K);
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
