// Expert permutation (A2): counts, offsets, sorted_slot, slot_pos.
//
// The position of routed slot s in expert group e is
//   offsets[e] + #{ s' < s : ids[s'] == e },
// i.e. a stable counting sort.  The rank inside a chunk of 256 slots is taken
// from per-wave 64-bit masks in LDS: lane l of wave w sets bit l of
// mask[w][e]; the slot's rank among same-expert slots of the chunk is the
// popcount of the masks of the lower waves plus the popcount of its own wave's
// mask below bit l.  Atomics only ever OR bits or add integer counts, so no
// result depends on timing.
//
// Two paths:
//  * T*K <= kSmallSlots: one workgroup does count, scan and scatter (decode);
//  * otherwise three kernels over tiles of kTileSlots slots: per-tile
//    histograms, a per-expert scan over tiles, and the scatter (every scatter
//    block re-derives the expert offsets from the per-expert totals).
// Both also write the compact list of non-empty groups, which the expert FFN
// uses to find the expert of a work unit with one load.
#include "moe_device.hpp"
#include "moe_internal.hpp"
#include "moe_route_permute.hpp"
#include "moe_topk.hpp"

namespace moe {

constexpr int kBlock = 256;           // 4 waves
constexpr int kChunk = 256;           // slots ranked at once
constexpr int kTileSlots = 4 * kChunk;
constexpr int kSmallSlots = 2048;
constexpr int kMaxE = 1024;
constexpr int kFuseBlock = 64 * kRouteFuseMaxT;  // one wave per token of the fused batch
static_assert(kRouteFuseMaxT * 32 <= kFuseBlock, "one slot per thread in the fused permutation");

// Ranks one chunk of up to 256 slots starting at c0 and scatters them; e is
// the expert id of this thread's slot c0 + tid (ignored past TK).  run[e]
// holds the next free position of group e and is advanced here.
__device__ void scatter_chunk(int e, int TK, int E, int c0,
                              unsigned long long (*masks)[kMaxE], int* run,
                              int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int s = c0 + tid;
  const bool in = s < TK;
  const bool ok = in && e >= 0 && e < E;
  const unsigned long long bit = 1ull << lane;
  if (ok) atomicOr(&masks[wv][e], bit);
  __syncthreads();
  int pos = -1;
  bool last = false;
  int tot = 0;
  if (ok) {
    int before = 0;
#pragma unroll
    for (int w2 = 0; w2 < kBlock / 64; ++w2) {
      const int c = __popcll(masks[w2][e]);
      before += (w2 < wv) ? c : 0;
      tot += c;
    }
    const int r = before + __popcll(masks[wv][e] & (bit - 1));
    pos = run[e] + r;
    last = (r == tot - 1);
    sorted_slot[pos] = s;
  }
  if (in) slot_pos[s] = pos;
  __syncthreads();
  if (ok) {
    masks[wv][e] = 0ull;
    if (last) run[e] += tot;
  }
  __syncthreads();
}

// groups[0] = number of non-empty groups, groups[1 + i] = the i-th of them in
// index order, -1 after the last.  cnt[] holds the group counts in LDS; wave 0
// compacts them.
__device__ void write_groups(const int* cnt, int G, int32_t* __restrict__ groups) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int base = 0;
  for (int c0 = 0; c0 < G; c0 += 64) {
    const int g = c0 + lane;
    const bool nz = g < G && cnt[g] > 0;
    const unsigned long long m = __ballot(nz);
    if (nz) groups[1 + base + __popcll(m & ((1ull << lane) - 1ull))] = g;
    base += __popcll(m);
  }
  if (lane == 0) groups[0] = base;
  for (int i = base + lane; i < G; i += 64) groups[1 + i] = -1;  // deterministic tail
}

// The shared group: slot T*K + t sits at position off_shared + t, both ways.
__device__ void write_shared_group(int T, int TK, int off_shared, int32_t* __restrict__ sorted_slot,
                                   int32_t* __restrict__ slot_pos, int first, int stride) {
  for (int t = first; t < T; t += stride) {
    sorted_slot[off_shared + t] = TK + t;
    slot_pos[TK + t] = off_shared + t;
  }
}

// Count, scan and scatter of all T*K slots by one 256-thread block.  `ids`
// may be global or LDS memory; masks and run are the block's LDS.  With
// init == true the LDS set-up is done here, else the caller has done it.
__device__ void permute_small_body(const int32_t* ids, int T, int E, int K, int has_shared,
                                   int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                   int32_t* __restrict__ sorted_slot,
                                   int32_t* __restrict__ slot_pos, int32_t* __restrict__ groups,
                                   unsigned long long (*masks)[kMaxE], int* run, int* wsum,
                                   bool init) {
  const int tid = threadIdx.x;
  const int TK = T * K, G = E + has_shared;
  // this thread's slot of the first chunk, loaded once (the whole input when
  // T*K <= 256), in flight during the LDS set-up
  const int id0 = tid < TK ? ids[tid] : -1;
  if (init) {
    for (int i = tid; i < (kBlock / 64) * kMaxE; i += kBlock) (&masks[0][0])[i] = 0ull;
    for (int e = tid; e < G; e += kBlock) run[e] = (e == E) ? T : 0;
    __syncthreads();
  }
  if (id0 >= 0 && id0 < E) atomicAdd(&run[id0], 1);
  for (int s = tid + kBlock; s < TK; s += kBlock) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&run[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < G; e += kBlock) counts[e] = run[e];
  write_groups(run, G, groups);
  __syncthreads();
  const int total = block_exclusive_scan<kBlock>(run, G, wsum);
  for (int e = tid; e < G; e += kBlock) offsets[e] = run[e];
  if (tid == 0) offsets[G] = total;
  const int off_shared = has_shared ? run[E] : 0;  // scatter_chunk only moves run[e < E]
  static_assert(kChunk == kBlock, "one slot per thread and chunk");
  for (int c0 = 0; c0 < TK; c0 += kChunk) {
    const int s = c0 + tid;
    scatter_chunk(c0 == 0 ? id0 : (s < TK ? ids[s] : -1), TK, E, c0, masks, run, sorted_slot, slot_pos);
  }
  if (has_shared) write_shared_group(T, TK, off_shared, sorted_slot, slot_pos, tid, kBlock);
}

__global__ __launch_bounds__(kBlock) void k_permute_small(
    const int32_t* __restrict__ ids, int T, int E, int K, int has_shared,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos,
    int32_t* __restrict__ groups) {
  __shared__ unsigned long long masks[kBlock / 64][kMaxE];
  __shared__ int run[kMaxE + 2];
  __shared__ int wsum[kBlock / 64];
  permute_small_body(ids, T, E, K, has_shared, counts, offsets, sorted_slot, slot_pos, groups,
                     masks, run, wsum, true);
}

// Router top-K and permutation of a batch of up to kRouteFuseMaxT tokens in
// one block of one wave per token (moe_route_permute.hpp): same outputs as
// the two kernels, one launch fewer.
template <int MAXV>
__global__ __launch_bounds__(kFuseBlock) void k_route_permute_small(
    const float* __restrict__ logits, int T, int E, int K, int has_shared,
    int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ groups) {
  __shared__ RpLds L;
  const RpOut o{ids, w, counts, offsets, sorted_slot, slot_pos, groups};
  rp_route<MAXV, kFuseBlock>(logits, T, E, K, has_shared, true, o, L);
  rp_permute<kFuseBlock>(T, E, K, has_shared, true, o, L);
}

// Tile histograms, written expert-major: cnt[e * ntiles + tile].
__global__ __launch_bounds__(kBlock) void k_permute_count(const int32_t* __restrict__ ids, int TK,
                                                         int E, int ntiles,
                                                         int32_t* __restrict__ cnt) {
  __shared__ int hist[kMaxE];
  const int tid = threadIdx.x, tile = blockIdx.x;
  for (int e = tid; e < E; e += kBlock) hist[e] = 0;
  __syncthreads();
  const int s0 = tile * kTileSlots, s1 = min(s0 + kTileSlots, TK);
  for (int s = s0 + tid; s < s1; s += kBlock) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kBlock) cnt[(size_t)e * ntiles + tile] = hist[e];
}

// Per expert: exclusive scan over tiles (in place) and the expert total.
__global__ __launch_bounds__(kBlock) void k_permute_scan_tiles(int32_t* __restrict__ cnt,
                                                              int ntiles,
                                                              int32_t* __restrict__ tot) {
  __shared__ int buf[kBlock];
  __shared__ int wsum[kBlock / 64];
  const int e = blockIdx.x, tid = threadIdx.x;
  int32_t* row = cnt + (size_t)e * ntiles;
  int carry = 0;
  for (int b0 = 0; b0 < ntiles; b0 += kBlock) {
    const int i = b0 + tid;
    buf[tid] = (i < ntiles) ? row[i] : 0;
    __syncthreads();
    const int sum = block_exclusive_scan<kBlock>(buf, kBlock, wsum);
    if (i < ntiles) row[i] = carry + buf[tid];
    carry += sum;
    __syncthreads();
  }
  if (tid == 0) tot[e] = carry;
}

__global__ __launch_bounds__(kBlock) void k_permute_scatter(
    const int32_t* __restrict__ ids, int T, int E, int K, int has_shared, int ntiles,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ tot,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos,
    int32_t* __restrict__ groups) {
  __shared__ unsigned long long masks[kBlock / 64][kMaxE];
  __shared__ int run[kMaxE + 2];
  __shared__ int wsum[kBlock / 64];
  const int tid = threadIdx.x, tile = blockIdx.x;
  const int TK = T * K, G = E + has_shared;
  for (int i = tid; i < (kBlock / 64) * kMaxE; i += kBlock) (&masks[0][0])[i] = 0ull;
  for (int e = tid; e < G; e += kBlock) run[e] = (e == E) ? T : tot[e];
  __syncthreads();
  if (tile == 0) {
    for (int e = tid; e < G; e += kBlock) counts[e] = run[e];
    write_groups(run, G, groups);
  }
  __syncthreads();
  const int total = block_exclusive_scan<kBlock>(run, G, wsum);
  if (tile == 0) {
    for (int e = tid; e < G; e += kBlock) offsets[e] = run[e];
    if (tid == 0) offsets[G] = total;
  }
  const int off_shared = has_shared ? run[E] : 0;
  for (int e = tid; e < E; e += kBlock) run[e] += cnt[(size_t)e * ntiles + tile];
  __syncthreads();
  const int s0 = tile * kTileSlots, s1 = min(s0 + kTileSlots, TK);
  for (int c0 = s0; c0 < s1; c0 += kChunk) {
    const int s = c0 + threadIdx.x;
    scatter_chunk(s < s1 ? ids[s] : -1, s1, E, c0, masks, run, sorted_slot, slot_pos);
  }
  if (has_shared)
    write_shared_group(T, TK, off_shared, sorted_slot, slot_pos, tile * kBlock + tid, ntiles * kBlock);
}

void register_permute_kernels(std::vector<const void*>& k) {
  k.push_back((const void*)&k_permute_small);
  k.push_back((const void*)&k_route_permute_small<1>);
  k.push_back((const void*)&k_route_permute_small<2>);
  k.push_back((const void*)&k_route_permute_small<4>);
  k.push_back((const void*)&k_route_permute_small<8>);
  k.push_back((const void*)&k_route_permute_small<16>);
  k.push_back((const void*)&k_permute_count);
  k.push_back((const void*)&k_permute_scan_tiles);
  k.push_back((const void*)&k_permute_scatter);
}

static inline int ntiles_of(int TK) { return (TK + kTileSlots - 1) / kTileSlots; }

size_t permute_workspace_bytes(int T, int E, int K) {
  const long TK = (long)T * K;
  if (TK <= kSmallSlots) return 0;
  return ((size_t)E * ntiles_of((int)TK) + (size_t)E) * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int K, int has_shared,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                          int32_t* slot_pos, int32_t* groups, void* ws, hipStream_t s) {
  const int TK = T * K;
  if (TK <= kSmallSlots) {
    MOE_LAUNCH("permute_small", s, k_permute_small, dim3(1), dim3(kBlock), 0, s, ids, T, E, K,
               has_shared, counts, offsets, sorted_slot, slot_pos, groups);
    return hipGetLastError();
  }
  const int nt = ntiles_of(TK);
  int32_t* cnt = (int32_t*)ws;
  int32_t* tot = cnt + (size_t)E * nt;
  MOE_LAUNCH("permute_count", s, k_permute_count, dim3(nt), dim3(kBlock), 0, s, ids, TK, E, nt, cnt);
  MOE_LAUNCH("permute_scan_tiles", s, k_permute_scan_tiles, dim3(E), dim3(kBlock), 0, s, cnt, nt, tot);
  MOE_LAUNCH("permute_scatter", s, k_permute_scatter, dim3(nt), dim3(kBlock), 0, s, ids, T, E, K,
             has_shared, nt, cnt, tot, counts, offsets, sorted_slot, slot_pos, groups);
  return hipGetLastError();
}

hipError_t launch_route_permute(const float* logits, int T, int E, int K, int has_shared,
                                int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                                int32_t* sorted_slot, int32_t* slot_pos, int32_t* groups, void* ws,
                                hipStream_t s) {
  if (T > kRouteFuseMaxT) {
    hipError_t e = launch_route_topk(logits, T, E, K, ids, w, s);
    if (e != hipSuccess) return e;
    return launch_permute(ids, T, E, K, has_shared, counts, offsets, sorted_slot, slot_pos,
                          groups, ws, s);
  }
#define MOE_RP(MAXV)                                                                           \
  MOE_LAUNCH("route_permute", s, (k_route_permute_small<MAXV>), dim3(1), dim3(kFuseBlock), 0, s, \
             logits, T, E, K, has_shared, ids, w, counts, offsets, sorted_slot, slot_pos, groups)
  if (E <= 64) MOE_RP(1);
  else if (E <= 128) MOE_RP(2);
  else if (E <= 256) MOE_RP(4);
  else if (E <= 512) MOE_RP(8);
  else MOE_RP(16);
#undef MOE_RP
  return hipGetLastError();
}

}  // namespace moe
