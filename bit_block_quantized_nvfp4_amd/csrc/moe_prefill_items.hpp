// Work items of the prefill grouped GEMMs: (group, 128-row tile of the
// group's sorted rows), ordered heaviest first, derived on the device from
// the group offsets (no device-to-host copy).
#pragma once

#include "moe_device.hpp"

namespace moe {

constexpr int kPM = 128;   // rows per tile
constexpr int kPK = 128;   // K per step
constexpr int kPMaxG = 1025;

struct PfTile {
  int g, p0, rows, nt;
};

// Item lookup from offsets.  Items are ordered heaviest first, so the short
// ones fill the end of the launch: class 0 holds the row tiles with 4 valid
// 32-row blocks (every full tile, and a last tile of more than 96 rows),
// classes 1, 2, 3 the last tiles with 3, 2, 1 valid blocks; within a class,
// group by group, row tile by row tile.  The four per-group counts are
// scanned at once as fields of one 64-bit word.  All threads
// must call it; false = no item.
// The 64-bit word moved by one DPP control (both halves; 0 where the control
// has no source lane or the row is masked off).
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long pf_dpp64(unsigned long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xF, false);
  return ((unsigned long long)hi << 32) | lo;
}
// Inclusive prefix sum of a 64-bit word over the 64 lanes, without LDS: row
// shifts by 1, 2, 4, 8, then row broadcasts of lanes 15 and 31.
__device__ __forceinline__ unsigned long long pf_wave_incl_scan64(unsigned long long v, int lane) {
  (void)lane;
  v += pf_dpp64<0x111, 0xF>(v);  // row_shr:1
  v += pf_dpp64<0x112, 0xF>(v);  // row_shr:2
  v += pf_dpp64<0x114, 0xF>(v);  // row_shr:4
  v += pf_dpp64<0x118, 0xF>(v);  // row_shr:8
  v += pf_dpp64<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += pf_dpp64<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Field k of a packed count word: class 0 (full tiles, up to S/128 + G) in
// bits [0, 31), classes 1..3 (at most one tile per group, G <= 1025) in 11
// bits each from bit 31 on.
__device__ __forceinline__ unsigned long long pf_unit(int k) {
  return k == 0 ? 1ull : 1ull << (31 + 11 * (k - 1));
}
__device__ __forceinline__ int pf_field(unsigned long long v, int k) {
  return k == 0 ? (int)(v & 0x7FFFFFFFull) : (int)((v >> (31 + 11 * (k - 1))) & 0x7FFull);
}

// Item of block b of nb when runs of R consecutive items go to one XCD:
// blocks are dealt to the 8 XCDs in turn (block b to XCD b % 8), so block
// (q R + r) 8 + x takes item (q 8 + x) R + r, i.e. XCD x runs items
// (q 8 + x) R .. + R - 1 back to back; the tail past the last whole run of
// 8 R blocks keeps item = block.  A bijection on [0, nb), and the items
// still start in about their list order.  Adjacent items of one group then
// share the XCD's L2 for their weight stream.
__device__ __forceinline__ int pf_item_of_block(int b, int nb, int R) {
  const int M = nb / (8 * R) * (8 * R);
  if (R <= 1 || b >= M) return b;
  const int x = b % 8, s = b / 8;
  return ((s / R) * 8 + x) * R + s % R;
}

template <int NTHR>
__device__ __forceinline__ bool pf_find_tile(const int32_t* __restrict__ offsets, int G, int NT,
                             unsigned long long* base, unsigned long long* wsum, PfTile* ti,
                             int xcd_run = 1) {
  constexpr int NWV = NTHR / 64;
  const int tid = threadIdx.x;
  for (int g = tid; g < G; g += NTHR) {
    const int cnt = offsets[g + 1] - offsets[g];
    const int rem = cnt % kPM;
    const int c0 = cnt / kPM + (rem > 96 ? 1 : 0);
    const int k = (rem > 0 && rem <= 96) ? 4 - (rem + 31) / 32 : 0;  // class of the last tile
    base[g] = (unsigned long long)c0 | (k ? pf_unit(k) : 0ull);
  }
  __syncthreads();
  const int per = (G + NTHR - 1) / NTHR;
  const int lo = min(tid * per, G), hi = min(lo + per, G);
  unsigned long long local = 0;
  for (int i = lo; i < hi; ++i) local += base[i];
  const int lane = tid & 63, wv = tid >> 6;
  const unsigned long long incl = pf_wave_incl_scan64(local, lane);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  unsigned long long before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    before += (i < wv) ? wsum[i] : 0ull;
    total += wsum[i];
  }
  unsigned long long run = before + incl - local;
  for (int i = lo; i < hi; ++i) {
    const unsigned long long v = base[i];
    base[i] = run;
    run += v;
  }
  __syncthreads();
  int L = pf_item_of_block(blockIdx.x, gridDim.x, xcd_run), k = 0;
  for (; k < 4; ++k) {
    const int n = pf_field(total, k) * NT;
    if (L < n) break;
    L -= n;
  }
  if (k == 4) return false;
  // last g with base_k[g] * NT <= L; groups with nothing in class k share the
  // base of the next group that has, so the search lands on the owner of L
  int lo_g = 0, hi_g = G - 1;
  while (lo_g < hi_g) {
    const int mid = (lo_g + hi_g + 1) >> 1;
    if (pf_field(base[mid], k) * NT <= L) lo_g = mid;
    else hi_g = mid - 1;
  }
  const int g = lo_g;
  const int cnt = offsets[g + 1] - offsets[g];
  const int li = L - pf_field(base[g], k) * NT;
  int nt, mt;
  if (k == 0) {
    const int mt_g = cnt / kPM + (cnt % kPM > 96 ? 1 : 0);
    nt = li / mt_g;
    mt = li % mt_g;
  } else {
    nt = li;
    mt = cnt / kPM;
  }
  ti->g = g;
  ti->nt = nt;
  ti->p0 = offsets[g] + mt * kPM;
  ti->rows = min(kPM, cnt - mt * kPM);
  return true;
}

}  // namespace moe
