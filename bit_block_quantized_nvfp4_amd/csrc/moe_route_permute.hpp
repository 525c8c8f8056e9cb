// Router top-K and permutation of a batch of up to kRouteFuseMaxT tokens by
// one block, kept in LDS (A1 + A2; used by k_route_permute_small and by the
// decode layer kernel, whose every block needs the routing of the batch).
//
//  * rp_route: every thread clears the group counts (the shared group holds
//    T) and the per-token expert bitmaps; wave t < T routes token t (the
//    router stage's rule, moe_topk.hpp) into LDS, and into the global ids / w
//    when `write`.  No barrier, so a caller can give its other waves other
//    work before rp_permute.
//  * rp_permute (every thread of the block): LDS atomics count the slots and
//    mark each slot's expert in its token's bitmap; one exclusive scan of
//    count | (count > 0) << 16, read straight from the counts, gives both the
//    group offsets (low 16 bits; at most kRouteFuseMaxT * 33 slots) and each
//    non-empty group's index in the compact list (high bits).  The rank of
//    slot s inside its group is the number of earlier slots with the same
//    expert (the stable counting sort of the multi-block path); the K experts
//    of one token are distinct, so that is the number of earlier tokens whose
//    bitmap holds the expert.  Leaves in LDS: cnt (counts), run (offset |
//    list index << 16), gl (the list), ss_l (the sorted slots); with `write`,
//    the permutation's global outputs too.
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
  int wsum[16];
  uint32_t bm[kRouteFuseMaxT][kRpMapWords];       // experts chosen by each token
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
    if (write)
      route_row_topk<MAXV>(logits + (size_t)wv * E, E, K, o.ids + (size_t)wv * K,
                           o.w + (size_t)wv * K, L.ids_l + wv * K);
    else
      route_row_topk<MAXV>(logits + (size_t)wv * E, E, K, L.ids_l + wv * K, L.w_l + wv * K);
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
  // rank of slot tid in its group: the earlier tokens that chose its expert
  int rank = 0;
  if (ok) {
#pragma unroll
    for (int u = 0; u + 1 < kRouteFuseMaxT; ++u)
      if (u < t_s) rank += (int)((L.bm[u][e_s >> 5] >> (e_s & 31)) & 1u);
  }
  // exclusive scan of count | (count > 0) << 16 over the G groups, PER
  // consecutive groups per thread
  constexpr int PER = (kRpMaxE + 1 + NT - 1) / NT;
  const int lo = tid * PER;
  int v[PER];
  int local = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int c = lo + p < G ? L.cnt[lo + p] : 0;
    v[p] = c | ((c > 0 ? 1 : 0) << 16);
    local += v[p];
  }
  const int incl = wave_incl_scan(local, lane);
  if (lane == 63) L.wsum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    before += (i < wv) ? L.wsum[i] : 0;
    total += L.wsum[i];
  }
  int run = before + incl - local;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int e = lo + p;
    if (e < G) {
      const int c = v[p] & 0xFFFF;
      L.run[e] = run;
      if (write) {
        o.counts[e] = c;
        o.offsets[e] = run & 0xFFFF;
      }
      if (c > 0) {
        L.gl[run >> 16] = e;
        if (write) o.groups[1 + (run >> 16)] = e;
      }
    }
    run += v[p];
  }
  const int nz = total >> 16;
  if (write) {
    for (int i = nz + tid; i < G; i += NT) o.groups[1 + i] = -1;  // deterministic tail
    if (tid == 0) {
      o.offsets[G] = total & 0xFFFF;
      o.groups[0] = nz;
    }
  }
  __syncthreads();
  if (tid < TK) {
    const int pos = ok ? (L.run[e_s] & 0xFFFF) + rank : -1;
    if (ok) {
      L.ss_l[pos] = tid;
      if (write) o.sorted_slot[pos] = tid;
    }
    if (write) o.slot_pos[tid] = pos;
  }
  if (has_shared) {  // slot T*K + t sits at position off + t, both ways
    const int off = L.run[E] & 0xFFFF;
    for (int t = tid; t < T; t += NT) {
      L.ss_l[off + t] = TK + t;
      if (write) {
        o.sorted_slot[off + t] = TK + t;
        o.slot_pos[TK + t] = off + t;
      }
    }
  }
  __syncthreads();
  return nz;
}

}  // namespace moe
