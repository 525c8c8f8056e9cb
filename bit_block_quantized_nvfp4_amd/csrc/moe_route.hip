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
#include "moe_xprep.hpp"

namespace moe {

template <int MAXV>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T,
                                                     int E, int K, int32_t* __restrict__ ids,
                                                     float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  route_row_topk<MAXV>(logits + (size_t)t * E, E, K, ids + (size_t)t * K, w + (size_t)t * K);
}

// Routing and the grouped path's activation prep in one launch: blocks
// [0, nr) route four tokens each, the next T blocks prepare activation arm a
// (rows of x into a.xh / a.unmul), and with a second arm (b.xh non-null) the T
// after those prepare arm b.  The two jobs read different inputs and write
// different outputs, so their blocks overlap on the GPU instead of running as
// two launches back to back.
template <int MAXV>
__global__ __launch_bounds__(256) void k_route_xprep(const float* __restrict__ logits, int T,
                                                      int E, int K, int32_t* __restrict__ ids,
                                                      float* __restrict__ w, int nr,
                                                      const uint16_t* __restrict__ x, int H,
                                                      XprepArm a, XprepArm b,
                                                      uint8_t* __restrict__ xq,
                                                      float* __restrict__ xs) {
  __shared__ float wmax[4];
  const int bid = blockIdx.x;
  if (bid < nr) {  // uniform per block
    const int t = bid * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform per wave
    route_row_topk<MAXV>(logits + (size_t)t * E, E, K, ids + (size_t)t * K, w + (size_t)t * K);
    return;
  }
  const int i = bid - nr;
  const XprepArm arm = i < T ? a : b;
  const int t = i < T ? i : i - T;
  if (arm.fp8)
    xprep_row<true>(x, H, t, arm.xh, arm.unmul, xq, xs, wmax);
  else
    xprep_row<false>(x, H, t, arm.xh, arm.unmul, xq, xs, wmax);
}

void register_route_kernels(std::vector<const void*>& k) {
  k.push_back((const void*)&k_route_topk<1>);
  k.push_back((const void*)&k_route_topk<2>);
  k.push_back((const void*)&k_route_topk<4>);
  k.push_back((const void*)&k_route_topk<8>);
  k.push_back((const void*)&k_route_topk<16>);
  k.push_back((const void*)&k_route_xprep<1>);
  k.push_back((const void*)&k_route_xprep<2>);
  k.push_back((const void*)&k_route_xprep<4>);
  k.push_back((const void*)&k_route_xprep<8>);
  k.push_back((const void*)&k_route_xprep<16>);
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

hipError_t launch_route_xprep(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                              const uint16_t* x, int H, XprepArm a, XprepArm b, uint8_t* xq,
                              float* xs, hipStream_t s) {
  const int nr = (T + 3) / 4;
  const dim3 grid((unsigned)(nr + (b.xh ? 2 * T : T))), block(256);
#define MOE_RX(MAXV)                                                                          \
  MOE_LAUNCH("route_xprep", s, (k_route_xprep<MAXV>), grid, block, 0, s, logits, T, E, K, ids, w, \
             nr, x, H, a, b, xq, xs)
  if (E <= 64) MOE_RX(1);
  else if (E <= 128) MOE_RX(2);
  else if (E <= 256) MOE_RX(4);
  else if (E <= 512) MOE_RX(8);
  else MOE_RX(16);
#undef MOE_RX
  return hipGetLastError();
}

}  // namespace moe
