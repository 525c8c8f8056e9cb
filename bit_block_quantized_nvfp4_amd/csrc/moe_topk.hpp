// Top-K of one token's logits by one wave64 (the router stage's rule): rank
// the experts by logit (larger first, equal logits -> lower index first, NaN
// counts as -inf), slot k = the rank-k expert, and weight the K selected
// experts by the softmax of their logits (equal to the full softmax
// restricted to the K and renormalised; the page "handover briefs", item A1
// and the indexer-selection kernel spec, give the rank rule).
//
// Lane l holds logits l, l+64, l+128, ... in registers and sorts its own keys
// once, largest first (a stable odd-even transposition sort, so equal keys
// stay in index order).  Each of the K rounds then takes one wave max over the
// 64 list heads (DPP inside rows of 16 lanes, row broadcasts across rows);
// the lane holding it pops its head.  When several heads hold the max, the
// lowest expert index wins (a wave min over those heads).  The weights are
// computed in fp32 with a fixed-order DPP sum.
#pragma once

#include <limits.h>
#include <math.h>

#include "moe_device.hpp"

namespace moe {

// Order-preserving 32-bit key of a logit: larger logit -> larger key; NaN was
// replaced by -inf; -0 is folded onto +0 so that equal logits have equal keys.
__device__ __forceinline__ uint32_t logit_key(float v) {
  const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// wave_max_u32 (moe_device.hpp) gives the max; the min below is used only on
// an exact tie.
// Min over the 64 lanes (the tie case only): quad and row steps as above,
// then readlane of lanes 0, 16, 32, 48.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp<0xB1>(v));
  v = min(v, dpp<0x4E>(v));
  v = min(v, dpp<0x141>(v));
  v = min(v, dpp<0x140>(v));
  const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return min(a, b);
}

// Route R tokens with one wave: rows[r] holds token r's E logits (global or
// LDS memory); tokens with live[r] false are skipped (uniform per wave).  Lane
// k < K writes slot k of ids[r] / w[r] (and of ids_copy[r] when given, e.g. an
// LDS copy for a consumer in the same block).  The R routes are independent
// and their steps are interleaved (measured: two routes per wave cost about
// two routes' time, so the kernels use R = 1).  Every lane of the wave must
// call it.
template <int MAXV, int R>
__device__ __forceinline__ void route_rows_topk(const float* const (&rows)[R], const bool (&live)[R],
                                                int E, int K, int32_t* const (&ids)[R],
                                                float* const (&w)[R],
                                                int32_t* const (&ids_copy)[R]) {
  const int lane = threadIdx.x & 63;
  uint32_t key[R][MAXV], jx[R][MAXV];  // key and slot j (expert lane + 64 j) of each entry
  // every load of a row is issued before the first is consumed: the index is
  // clamped into the row (E >= 1) instead of guarding each load, which would
  // make each one a separate round trip to memory
  float zr[R][MAXV];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (live[r]) {  // uniform per wave
#pragma unroll
      for (int j = 0; j < MAXV; ++j) zr[r][j] = rows[r][min(lane + 64 * j, E - 1)];
    } else {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) zr[r][j] = -INFINITY;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
      const int e = lane + 64 * j;
      const bool in = live[r] && e < E;
      const float z = zr[r][j];
      // absent elements get key 0, below every real key (-inf maps to 0x007FFFFF)
      key[r][j] = in ? logit_key((z != z) ? -INFINITY : z) : 0u;
      jx[r][j] = (uint32_t)j;
    }
  // largest key first; a swap only on a strictly larger key keeps equal keys
  // in ascending j, i.e. ascending expert index
#pragma unroll
  for (int pass = 0; pass < MAXV; ++pass) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = pass & 1; i + 1 < MAXV; i += 2) {
        const bool sw = key[r][i + 1] > key[r][i];
        const uint32_t k0 = key[r][i], k1 = key[r][i + 1], j0 = jx[r][i], j1 = jx[r][i + 1];
        key[r][i] = sw ? k1 : k0;
        key[r][i + 1] = sw ? k0 : k1;
        jx[r][i] = sw ? j1 : j0;
        jx[r][i + 1] = sw ? j0 : j1;
      }
  }

  float zsel[R];
  int isel[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    zsel[r] = -INFINITY;
    isel[r] = 0;
  }
  for (int k = 0; k < K; ++k) {
    uint32_t kmax[R];
#pragma unroll
    for (int r = 0; r < R; ++r) kmax[r] = wave_max_u32(key[r][0]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool has = key[r][0] == kmax[r];
      const unsigned long long m = __ballot(has);
      int win;  // expert index of the winner
      if (__popcll(m) == 1) {
        const int wl = __ffsll((long long)m) - 1;
        win = wl + 64 * __builtin_amdgcn_readlane((int)jx[r][0], wl);
      } else {
        win = (int)wave_min_u32(has ? (uint32_t)lane + 64u * jx[r][0] : 0xFFFFFFFFu);
      }
      if (lane == k) {
        zsel[r] = key_logit(kmax[r]);
        isel[r] = win;
      }
      if (lane == (win & 63)) {  // pop the head: the next largest becomes the head
#pragma unroll
        for (int i = 0; i + 1 < MAXV; ++i) {
          key[r][i] = key[r][i + 1];
          jx[r][i] = jx[r][i + 1];
        }
        key[r][MAXV - 1] = 0u;
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float z0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zsel[r]), 0));
    float ex = 0.f;
    if (lane < K) ex = expf(zsel[r] == z0 ? 0.f : zsel[r] - z0);
    const float sum = wave_sum_dpp(ex);
    if (live[r] && lane < K) {
      ids[r][lane] = isel[r];
      w[r][lane] = ex / sum;
      if (ids_copy[r]) ids_copy[r][lane] = isel[r];
    }
  }
}

// Route one token (route_rows_topk with R = 1).
template <int MAXV>
__device__ __forceinline__ void route_row_topk(const float* row, int E, int K, int32_t* ids_t,
                                               float* w_t, int32_t* ids_copy = nullptr) {
  const float* const rows[1] = {row};
  const bool live[1] = {true};
  int32_t* const ids[1] = {ids_t};
  float* const ws[1] = {w_t};
  int32_t* const cp[1] = {ids_copy};
  route_rows_topk<MAXV, 1>(rows, live, E, K, ids, ws, cp);
}

}  // namespace moe
