// Router top-K and permutation of a batch of up to kRouteFuseMaxT tokens by
// one block, kept in LDS (A1 + A2; used by k_route_permute_small and by the
// decode layer kernel, whose every block needs the routing of the batch).
//
//  * rp_route: every thread clears the group counts (the shared group holds
//    T); wave t < T routes token t (the router stage's rule, moe_topk.hpp)
//    into LDS, and into the global ids / w when `write`.  No barrier, so a
//    caller can give its other waves other work before rp_permute.
//  * rp_permute (every thread of the block): LDS atomics count the slots;
//    one exclusive scan of count | (count > 0) << 16 gives both the group
//    offsets (low 16 bits; at most kRouteFuseMaxT * 33 slots) and each
//    non-empty group's index in the compact list (high bits); the rank of
//    slot s inside its group is the number of earlier slots with the same
//    expert, counted from the ids in LDS (the stable counting sort of the
//    multi-block path, without its per-chunk masks).  Leaves in LDS: cnt
//    (counts), run (offset | list index << 16), gl (the list), ss_l (the
//    sorted slots); with `write`, the permutation's global outputs too.
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

struct RpLds {
  int cnt[kRpMaxE + 1];
  int run[kRpMaxE + 1];
  int gl[kRpMaxE + 1];
  int wsum[16];
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
  const int tid = threadIdx.x;
  const int G = E + has_shared, TK = T * K;
  __syncthreads();
  const int e_s = tid < TK ? L.ids_l[tid] : -1;
  const bool ok = e_s >= 0 && e_s < E;
  if (ok) atomicAdd(&L.cnt[e_s], 1);
  __syncthreads();
  for (int e = tid; e < G; e += NT) {
    const int c = L.cnt[e];
    if (write) o.counts[e] = c;
    L.run[e] = c | ((c > 0 ? 1 : 0) << 16);
  }
  __syncthreads();
  const int packed = block_exclusive_scan<NT>(L.run, G, L.wsum);
  const int nz = packed >> 16;
  for (int e = tid; e < G; e += NT) {
    const int v = L.run[e];
    if (write) o.offsets[e] = v & 0xFFFF;
    if (L.cnt[e] > 0) {
      L.gl[v >> 16] = e;
      if (write) o.groups[1 + (v >> 16)] = e;
    }
  }
  if (write) {
    for (int i = nz + tid; i < G; i += NT) o.groups[1 + i] = -1;  // deterministic tail
    if (tid == 0) {
      o.offsets[G] = packed & 0xFFFF;
      o.groups[0] = nz;
    }
  }
  if (tid < TK) {
    int pos = -1;
    if (ok) {
      int r = 0;
      const int s4 = tid & ~3;
      for (int j = 0; j < s4; j += 4) {
        const int4 v = *(const int4*)(L.ids_l + j);
        r += (v.x == e_s) + (v.y == e_s) + (v.z == e_s) + (v.w == e_s);
      }
      for (int j = s4; j < tid; ++j) r += L.ids_l[j] == e_s;
      pos = (L.run[e_s] & 0xFFFF) + r;
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
