// Router top-K and permutation of a batch of up to kRouteFuseMaxT tokens by
// one block, kept in LDS (A1 + A2; used by k_route_permute_small and by the
// decode layer kernel, whose every block needs the routing of the batch).
//
//  * rp_route: every thread clears the group counts (the shared group holds
//    T) and the per-token expert bitmaps; wave t < T routes token t (the
//    router stage's rule, moe_topk.hpp) into LDS, and into the global ids / w
//    when `write`.  No barrier, so a caller can give its other waves other
//    work before rp_permute.
//  * rp_permute (every thread of the block) places the routed slots in the
//    stable counting-sort order of the multi-block path without a scan over
//    the groups: LDS atomics count the slots per expert and mark each slot's
//    expert in its token's bitmap; one wave then takes, per 32-expert word,
//    the number of slots (the tokens' bitmap populations) and of distinct
//    experts (the union's population), and their exclusive prefixes over the
//    words.  A slot with expert e then finds the slots of smaller experts
//    (the word prefix plus the tokens' bits below e in e's word), its rank
//    among the slots of e (the earlier tokens whose bitmap holds e: the K
//    experts of a token are distinct) and e's index in the compact list (the
//    same from the union).  Leaves in LDS: cnt (counts), run (offset | list
//    index << 16) and gl (the list) for the active groups, ss_l (the sorted
//    slots); with `write`, the permutation's global outputs for every group.
#pragma once

#include "moe_device.hpp"
#include "moe_internal.hpp"
#include "moe_topk.hpp"

namespace moe {

constexpr int kRpMaxE = 1024;
constexpr int kRpMaxSlots = kRouteFuseMaxT * 32;  // routed slots of the batch (K <= 32)

// Exclusive scan, in place, of a[0..n) held in LDS, by a block of NT threads.
// Returns the total.  Must be called by every thread of the block.
template <int NT>
__device__ int block_exclusive_scan(int* a, int n, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n + NT - 1) / NT;
  const int lo = min(tid * per, n), hi = min(lo + per, n);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += a[i];
  const int incl = wave_incl_scan(local, lane);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    before += (i < wv) ? wsum[i] : 0;
    total += wsum[i];
  }
  int run = before + incl - local;
  for (int i = lo; i < hi; ++i) {
    const int v = a[i];
    a[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

constexpr int kRpMapWords = kRpMaxE / 32;         // bitmap words per token

struct RpLds {
  int cnt[kRpMaxE + 1];
  int run[kRpMaxE + 1];
  int gl[kRpMaxE + 1];
  uint32_t bm[kRouteFuseMaxT][kRpMapWords];       // experts chosen by each token
  uint32_t un[kRpMapWords];                       // their union
  int pre_s[kRpMapWords + 1];                     // slots of experts in words < w
  int pre_g[kRpMapWords + 1];                     // distinct experts in words < w
  __align__(16) int32_t ids_l[kRpMaxSlots];
  float w_l[kRpMaxSlots];
  int32_t ss_l[kRpMaxSlots + kRouteFuseMaxT];
};

template <int MAXV, int NT>
__device__ __forceinline__ void rp_route(const float* __restrict__ logits, int T, int E, int K,
                                         int has_shared, bool write, const RpOut& o, RpLds& L) {
  static_assert(NT >= 64 * kRouteFuseMaxT && NT >= kRpMaxSlots, "a wave per token, a thread per slot");
  const int tid = threadIdx.x, wv = tid >> 6;
  const int G = E + has_shared;
  for (int e = tid; e < G; e += NT) L.cnt[e] = (e == E) ? T : 0;
  for (int i = tid; i < kRouteFuseMaxT * kRpMapWords; i += NT) (&L.bm[0][0])[i] = 0u;
  if (wv < T) {  // uniform per wave
    // the routing waves first on their SIMDs (the decode layer kernel's row
    // converting waves share them): T=8 layer 42.0 -> 41.75 us, T=4 29.5 -> 29.3
    __builtin_amdgcn_s_setprio(3);
    if (write)
      route_row_topk<MAXV>(logits + (size_t)wv * E, E, K, o.ids + (size_t)wv * K,
                           o.w + (size_t)wv * K, L.ids_l + wv * K);
    else
      route_row_topk<MAXV>(logits + (size_t)wv * E, E, K, L.ids_l + wv * K, L.w_l + wv * K);
    __builtin_amdgcn_s_setprio(0);
  }
}

template <int NT>
__device__ __forceinline__ int rp_permute(int T, int E, int K, int has_shared, bool write,
                                          const RpOut& o, RpLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = E + has_shared, TK = T * K;
  __syncthreads();  // the routed ids, the cleared counts and bitmaps
  const int e_s = tid < TK ? L.ids_l[tid] : -1;
  const bool ok = e_s >= 0 && e_s < E;
  const int t_s = tid < TK ? tid / K : 0;
  if (ok) {
    atomicAdd(&L.cnt[e_s], 1);
    atomicOr(&L.bm[t_s][e_s >> 5], 1u << (e_s & 31));
  }
  __syncthreads();
  if (wv == 0) {  // per word: slots and distinct experts, exclusive prefixes
    uint32_t u = 0u;
    int ns = 0;
    if (lane < kRpMapWords) {
#pragma unroll
      for (int t = 0; t < kRouteFuseMaxT; ++t)
        if (t < T) {
          const uint32_t m = L.bm[t][lane];
          u |= m;
          ns += __popc(m);
        }
      L.un[lane] = u;
    }
    const int ng = __popc(u);
    const int is = wave_incl_scan(ns, lane), ig = wave_incl_scan(ng, lane);
    if (lane <= kRpMapWords) {  // lane 32 holds the totals
      L.pre_s[lane] = is - ns;
      L.pre_g[lane] = ig - ng;
    }
  }
  // rank of slot tid in its group: the earlier tokens that chose its expert
  int rank = 0;
  if (ok) {
#pragma unroll
    for (int u = 0; u + 1 < kRouteFuseMaxT; ++u)
      if (u < t_s) rank += (int)((L.bm[u][e_s >> 5] >> (e_s & 31)) & 1u);
  }
  __syncthreads();
  // slots of experts below e (e < E)
  auto slots_below = [&](int e) {
    const int w = e >> 5;
    const uint32_t below = (1u << (e & 31)) - 1u;
    int c = L.pre_s[w];
#pragma unroll
    for (int t = 0; t < kRouteFuseMaxT; ++t)
      if (t < T) c += __popc(L.bm[t][w] & below);
    return c;
  };
  const int nzr = L.pre_g[kRpMapWords], tkv = L.pre_s[kRpMapWords];
  const int nz = nzr + has_shared;
  if (tid < TK) {
    int pos = -1;
    if (ok) {
      const int off = slots_below(e_s);
      pos = off + rank;
      L.ss_l[pos] = tid;
      if (write) o.sorted_slot[pos] = tid;
      if (rank == 0) {  // the group's first slot publishes the group
        const int w = e_s >> 5;
        const int li = L.pre_g[w] + __popc(L.un[w] & ((1u << (e_s & 31)) - 1u));
        L.gl[li] = e_s;
        L.run[e_s] = off | (li << 16);
        if (write) o.groups[1 + li] = e_s;
      }
    }
    if (write) o.slot_pos[tid] = pos;
  }
  if (has_shared) {  // the shared group is the last one; slot T*K + t at tkv + t
    if (tid == 0) {
      L.gl[nzr] = E;
      L.run[E] = tkv | (nzr << 16);
      if (write) o.groups[1 + nzr] = E;
    }
    for (int t = tid; t < T; t += NT) {
      L.ss_l[tkv + t] = TK + t;
      if (write) {
        o.sorted_slot[tkv + t] = TK + t;
        o.slot_pos[TK + t] = tkv + t;
      }
    }
  }
  if (write) {  // counts and offsets of every group, the list's tail
    for (int e = tid; e < G; e += NT) {
      o.counts[e] = L.cnt[e];
      o.offsets[e] = e < E ? slots_below(e) : tkv;
    }
    for (int i = nz + tid; i < G; i += NT) o.groups[1 + i] = -1;  // deterministic tail
    if (tid == 0) {
      o.offsets[G] = tkv + (has_shared ? T : 0);
      o.groups[0] = nz;
    }
  }
  __syncthreads();
  return nz;
}

}  // namespace moe
