// Expert FFN of the NVFP4 MoE layer (A3-A9): per-row e4m3 activation
// quantisation, the decode multi-row GEMV and the prefill grouped GEMM.
//
// Numerics (the table attributing the transposed-MoE perplexity gap in the
// issue "[job] Qwen3.8-Flash-Next: long-context cold prefill to SGLang
// parity"): weights are dequantised as e2m1 x e4m3 block scale (exact in bf16:
// at most 6 significant bits, exponents 2^-10 .. 2^12), the products run on
// bf16 MFMA with f32 accumulation, scale2 (and the FP8 row scale) multiply the
// f32 sums, SiLU(gate) * up is stored as bf16, the down output is stored as
// bf16 per sorted slot.
//
// NVFP4 operand layout in registers: a lane reads 16 bytes (32 codes, element
// 2j in the low nibble of byte j) of one weight row and turns each 32-bit word
// into one 8-element bf16 MFMA operand: v_cvt_scalef32_pk_f32_fp4 gives the
// two e2m1 values of a byte, one f32 multiply per value applies the e4m3 block
// scale (the converter's own scale operand only carries a power of two), and
// v_cvt_pk_bf16_f32 packs the pair.  The activation operand of the same MFMA
// lane is read with the same K order, so the dot products run over a
// permutation of K that both operands share.
#include <math.h>

#include "moe_ffn_common.hpp"
#include "moe_internal.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Per-token-row e4m3 quantisation (FP8 arm, option (a) of the issue above):
// s_t = absmax/448, q = e4m3_rne_sat(x * (448/absmax)); an all-zero row takes
// s_t = 1.  One 256-thread block per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rowquant_e4m3(const uint16_t* __restrict__ x, int H,
                                                       uint8_t* __restrict__ xq,
                                                       float* __restrict__ xs) {
  __shared__ float wmax[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const u32x4* row = (const u32x4*)(x + (size_t)t * H);
  float amax = 0.f;
  for (int c = tid; c < H / 8; c += 256) {
    const u32x4 v = row[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[j] & 0xFFFFu)));
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[j] >> 16)));
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
  if (tid == 0) xs[t] = s;
  u32x2* out = (u32x2*)(xq + (size_t)t * H);
  for (int c = tid; c < H / 8; c += 256) {
    const u32x4 v = row[c];
    u32x2 o;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float f0 = bf16_bits_to_f32(v[2 * j] & 0xFFFFu) * inv;
      float f1 = bf16_bits_to_f32(v[2 * j] >> 16) * inv;
      float f2 = bf16_bits_to_f32(v[2 * j + 1] & 0xFFFFu) * inv;
      float f3 = bf16_bits_to_f32(v[2 * j + 1] >> 16) * inv;
      f0 = fminf(fmaxf(f0, -448.f), 448.f);
      f1 = fminf(fmaxf(f1, -448.f), 448.f);
      f2 = fminf(fmaxf(f2, -448.f), 448.f);
      f3 = fminf(fmaxf(f3, -448.f), 448.f);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, w, true);
      o[j] = (uint32_t)w;
    }
    out[c] = o;
  }
}

// ---------------------------------------------------------------------------
// Prefill path: grouped GEMM on 32x32x16 bf16 MFMA.
//
// A work item is (group, 128-row tile of its sorted rows, N tile).  Items are
// enumerated group by group, N tile by N tile, row tile by row tile, and block
// b takes item remap(b) so that the blocks of one XCD (b % 8) hold a
// contiguous run of items: the row tiles that reuse one weight tile share that
// XCD's L2.  Each block re-derives the item table from offsets in LDS, so no
// device-to-host copy or planning launch is needed.
//
// The activation tile (128 rows x 128 K, bf16) is staged in LDS with a 16-byte
// row pad and double-buffered; each wave dequantises only its own weight rows
// in registers (no weight tile is dequantised twice in a block).
// Lane (n = l%32, q = l/32): weight row n of an MFMA block; in K step s its
// 16-byte load c (c = 0, 1) covers elements 128s + 64c + 32q + [0, 32), word w
// of it feeds sub-step 4c + w; activations are read in the same order.
// ---------------------------------------------------------------------------
constexpr int kBM = 128;           // rows per tile
constexpr int kKS = 128;           // K per step
constexpr int kLDA = kKS + 8;      // padded LDS row (bf16 elements)
constexpr int kMaxG = 1025;

__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb / 8, r = nb % 8, xcd = b % 8, i = b / 8;
  return (xcd < r) ? xcd * (q + 1) + i : r * (q + 1) + (xcd - r) * q + i;
}

struct TileInfo {
  int g, p0, rows, nt;
};

// Work item lookup. All threads of the block must call it. Returns false if
// the block has no item.
__device__ bool find_tile(const int32_t* __restrict__ offsets, int G, int NT, int* base, int* wsum,
                          TileInfo* ti) {
  const int tid = threadIdx.x;
  for (int g = tid; g < G; g += 256) {
    const int cnt = offsets[g + 1] - offsets[g];
    base[g] = cnt > 0 ? (cnt + kBM - 1) / kBM : 0;
  }
  __syncthreads();
  // exclusive scan of tile counts
  const int per = (G + 255) / 256;
  const int lo = min(tid * per, G), hi = min(lo + per, G);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += base[i];
  const int lane = tid & 63, wv = tid >> 6;
  const int incl = wave_incl_scan(local, lane);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int i = 0; i < 4; ++i) {
    before += (i < wv) ? wsum[i] : 0;
    total += wsum[i];
  }
  int run = before + incl - local;
  for (int i = lo; i < hi; ++i) {
    const int v = base[i];
    base[i] = run;
    run += v;
  }
  __syncthreads();
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  if (L >= total * NT) return false;
  // binary search: last g with base[g] * NT <= L and a non-empty range
  int lo_g = 0, hi_g = G - 1;
  while (lo_g < hi_g) {
    const int mid = (lo_g + hi_g + 1) >> 1;
    if (base[mid] * NT <= L) lo_g = mid;
    else hi_g = mid - 1;
  }
  // groups with zero tiles share the base of the next non-empty group; step
  // forward to the one that owns L
  int g = lo_g;
  const int mt_g = ((offsets[g + 1] - offsets[g]) + kBM - 1) / kBM;
  const int local_i = L - base[g] * NT;
  const int nt = local_i / mt_g, mt = local_i % mt_g;
  ti->g = g;
  ti->p0 = offsets[g] + mt * kBM;
  ti->rows = min(kBM, offsets[g + 1] - ti->p0);
  ti->nt = nt;
  return true;
}

// Stage one 128 x 128 activation tile (gathered x rows, or contiguous h rows)
// into registers: thread tid covers 16-byte chunk tid%16 of rows tid/16 + 16j.
template <bool FP8>
__device__ __forceinline__ void load_a_rows(u32x4 (&buf)[8], const uint16_t* __restrict__ src,
                                            const uint8_t* __restrict__ srcq, const int* rowidx,
                                            int ld, int k0) {
  const int c = threadIdx.x & 15, r0 = threadIdx.x >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int ri = rowidx[r0 + 16 * j];
    if (ri >= 0) {
      if (FP8) {
        const u32x2 v = *(const u32x2*)(srcq + (size_t)ri * ld + k0 + 8 * c);
        buf[j] = __builtin_bit_cast(u32x4, fp8x8_to_bf16(v));
      } else {
        buf[j] = *(const u32x4*)(src + (size_t)ri * ld + k0 + 8 * c);
      }
    } else {
      buf[j] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void store_a_rows(const u32x4 (&buf)[8], uint16_t (*As)[kLDA]) {
  const int c = threadIdx.x & 15, r0 = threadIdx.x >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) *(u32x4*)(&As[r0 + 16 * j][8 * c]) = buf[j];
}

// Weight codes + scales of one K step for one 32-row MFMA block.
struct WStep {
  u32x4 c[2];
  uint32_t s[2];
};

__device__ __forceinline__ void load_w_step(WStep& w, const uint8_t* __restrict__ codes_row,
                                            const uint8_t* __restrict__ scales_row, int s, int q) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    w.c[c] = *(const u32x4*)(codes_row + 64 * s + 32 * c + 16 * q);
    w.s[c] = *(const uint16_t*)(scales_row + 8 * s + 4 * c + 2 * q);
  }
}

// One K step of MFMAs for NMB row blocks x NB weight blocks.
template <int NB>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[4][NB], const WStep (&w)[NB],
                                         uint16_t (*As)[kLDA], int nmb) {
  const int lane = threadIdx.x & 63, m = lane & 31, q = lane >> 5;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float sc[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      sc[nb][0] = e4m3_to_f32(w[nb].s[c] & 0xFFu);
      sc[nb][1] = e4m3_to_f32(w[nb].s[c] >> 8);
    }
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      bf16x8 bv[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) bv[nb] = dq8(w[nb].c[c][wd], sc[nb][wd >> 1]);
      const int kcol = 64 * c + 32 * q + 8 * wd;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < nmb) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4*)(&As[32 * mb + m][kcol]));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[nb], acc[mb][nb], 0, 0, 0);
        }
      }
    }
  }
}

// gate_up + SiLU: N tile = 128 gate/up pairs; wave w owns pairs [32w, 32w+32)
// as two MFMA blocks (gate rows, up rows).
template <bool FP8>
__global__ __launch_bounds__(256, 2) void k_grouped_gate_up(
    const uint8_t* __restrict__ gu_codes, const uint8_t* __restrict__ gu_scales,
    const float* __restrict__ scale2, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slot, int T, int K,
    int H, int I, int G, int has_shared, uint16_t* __restrict__ h) {
  __shared__ uint16_t As[2][kBM][kLDA];
  __shared__ int base[kMaxG];
  __shared__ int wsum[4];
  __shared__ int tok_s[kBM];
  TileInfo ti;
  if (!find_tile(offsets, G, I / 128, base, wsum, &ti)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int r = tid; r < kBM; r += 256)
    tok_s[r] = (r < ti.rows) ? slot_token(sorted_slot[ti.p0 + r], T, K, has_shared) : -1;
  __syncthreads();

  const int e = ti.g, nmb = (ti.rows + 31) / 32;
  const int n32 = lane & 31, q = lane >> 5;
  const size_t rowb = (size_t)H / 2, srow = (size_t)H / 16;
  const size_t grow = (size_t)e * 2 * I + (size_t)ti.nt * 128 + wv * 32 + n32;
  const uint8_t* crow[2] = {gu_codes + grow * rowb, gu_codes + (grow + I) * rowb};
  const uint8_t* srw[2] = {gu_scales + grow * srow, gu_scales + (grow + I) * srow};
  const int nsteps = H / kKS;

  f32x16 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{};

  u32x4 abuf[8];
  WStep wcur[2], wnext[2];
  load_a_rows<FP8>(abuf, x, xq, tok_s, H, 0);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) load_w_step(wcur[nb], crow[nb], srw[nb], 0, q);
  store_a_rows(abuf, As[0]);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    if (s + 1 < nsteps) {
      load_a_rows<FP8>(abuf, x, xq, tok_s, H, (s + 1) * kKS);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) load_w_step(wnext[nb], crow[nb], srw[nb], s + 1, q);
    }
    mma_step<2>(acc, wcur, As[cur], nmb);
    if (s + 1 < nsteps) {
      store_a_rows(abuf, As[cur ^ 1]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) wcur[nb] = wnext[nb];
    }
    __syncthreads();
  }

  const float s2g = scale2[3 * e + 0], s2u = scale2[3 * e + 1];
  const int col = ti.nt * 128 + wv * 32 + n32;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb < nmb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * mb + 8 * (i >> 2) + 4 * q + (i & 3);
        const int tk = tok_s[r];
        if (r < ti.rows && tk >= 0) {
          const float rs = FP8 ? xs[tk] : 1.0f;
          const float g = acc[mb][0][i] * s2g * rs, u = acc[mb][1][i] * s2u * rs;
          h[(size_t)(ti.p0 + r) * I + col] = f32_to_bf16_bits(silu_f32(g) * u);
        }
      }
    }
  }
}

// down: N tile = 256 output rows; wave w owns rows [64w, 64w+64) as two MFMA
// blocks; A = h rows of the tile (contiguous sorted positions).
__global__ __launch_bounds__(256, 2) void k_grouped_down(
    const uint8_t* __restrict__ dn_codes, const uint8_t* __restrict__ dn_scales,
    const float* __restrict__ scale2, const uint16_t* __restrict__ h,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slot, int T, int K,
    int H, int I, int G, int has_shared, uint16_t* __restrict__ y) {
  __shared__ uint16_t As[2][kBM][kLDA];
  __shared__ int base[kMaxG];
  __shared__ int wsum[4];
  __shared__ int row_s[kBM];
  TileInfo ti;
  if (!find_tile(offsets, G, H / 256, base, wsum, &ti)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int r = tid; r < kBM; r += 256)
    row_s[r] = (r < ti.rows && slot_token(sorted_slot[ti.p0 + r], T, K, has_shared) >= 0)
                   ? ti.p0 + r
                   : -1;
  __syncthreads();

  const int e = ti.g, nmb = (ti.rows + 31) / 32;
  const int n32 = lane & 31, q = lane >> 5;
  const size_t rowb = (size_t)I / 2, srow = (size_t)I / 16;
  const size_t r0 = (size_t)e * H + (size_t)ti.nt * 256 + wv * 64 + n32;
  const uint8_t* crow[2] = {dn_codes + r0 * rowb, dn_codes + (r0 + 32) * rowb};
  const uint8_t* srw[2] = {dn_scales + r0 * srow, dn_scales + (r0 + 32) * srow};
  const int nsteps = I / kKS;

  f32x16 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{};

  u32x4 abuf[8];
  WStep wcur[2], wnext[2];
  load_a_rows<false>(abuf, h, nullptr, row_s, I, 0);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) load_w_step(wcur[nb], crow[nb], srw[nb], 0, q);
  store_a_rows(abuf, As[0]);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    if (s + 1 < nsteps) {
      load_a_rows<false>(abuf, h, nullptr, row_s, I, (s + 1) * kKS);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) load_w_step(wnext[nb], crow[nb], srw[nb], s + 1, q);
    }
    mma_step<2>(acc, wcur, As[cur], nmb);
    if (s + 1 < nsteps) {
      store_a_rows(abuf, As[cur ^ 1]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) wcur[nb] = wnext[nb];
    }
    __syncthreads();
  }

  const float s2d = scale2[3 * e + 2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb < nmb) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = ti.nt * 256 + wv * 64 + nb * 32 + n32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * mb + 8 * (i >> 2) + 4 * q + (i & 3);
          if (r < ti.rows && row_s[r] >= 0)
            y[(size_t)(ti.p0 + r) * H + col] = f32_to_bf16_bits(acc[mb][nb][i] * s2d);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
void register_ffn_kernels(std::vector<const void*>& k) {
  k.push_back((const void*)&k_rowquant_e4m3);
  k.push_back((const void*)&k_grouped_gate_up<false>);
  k.push_back((const void*)&k_grouped_gate_up<true>);
  k.push_back((const void*)&k_grouped_down);
  register_decode_kernels(k);
}

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t ffn_workspace_bytes(int T, int K, int H, int I, int has_shared, int act_mode) {
  const size_t S = (size_t)T * K + (has_shared ? (size_t)T : 0);
  size_t b = align256(S * I * sizeof(uint16_t));
  if (act_mode == MOE_ACT_FP8_ROW) b += align256((size_t)T * H) + align256((size_t)T * sizeof(float));
  if (T <= kDecodeMaxT && decode_supported(H, I)) b += decode_workspace_extra(T, H);
  return b;
}

hipError_t launch_expert_ffn(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                             const int32_t* offsets, const int32_t* sorted_slot,
                             const int32_t* groups, int act_mode, uint16_t* y, void* ws,
                             hipStream_t s) {
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const int G = W.E + hs;
  const size_t S = (size_t)T * K + (hs ? (size_t)T : 0);
  uint8_t* wp = (uint8_t*)ws;
  uint16_t* hbuf = (uint16_t*)wp;
  wp += align256(S * I * sizeof(uint16_t));
  uint8_t* xq = nullptr;
  float* xs = nullptr;
  const bool fp8 = act_mode == MOE_ACT_FP8_ROW;
  if (fp8) {
    xq = wp;
    wp += align256((size_t)T * H);
    xs = (float*)wp;
    wp += align256((size_t)T * sizeof(float));
  }
  if (T <= kDecodeMaxT && decode_supported(H, I))
    return launch_decode_ffn(W, x, T, K, offsets, sorted_slot, groups, fp8, hbuf, xq, xs, wp, y, s);
  if (fp8) MOE_LAUNCH("rowquant_e4m3", s, k_rowquant_e4m3, dim3(T), dim3(256), 0, s, x, H, xq, xs);
  // grouped GEMM: at most S/kBM full tiles plus one partial tile per group
  const long mt_bound = (long)S / kBM + G;
  const dim3 blk(256);
  const dim3 g1((unsigned)(mt_bound * (I / 128)));
  if (fp8)
    MOE_LAUNCH("grouped_gate_up", s, (k_grouped_gate_up<true>), g1, blk, 0, s, W.gu_codes,
               W.gu_scales, W.scale2, x, xq, xs, offsets, sorted_slot, T, K, H, I, G, hs, hbuf);
  else
    MOE_LAUNCH("grouped_gate_up", s, (k_grouped_gate_up<false>), g1, blk, 0, s, W.gu_codes,
               W.gu_scales, W.scale2, x, xq, xs, offsets, sorted_slot, T, K, H, I, G, hs, hbuf);
  const dim3 g2((unsigned)(mt_bound * (H / 256)));
  MOE_LAUNCH("grouped_down", s, k_grouped_down, g2, blk, 0, s, W.dn_codes, W.dn_scales, W.scale2,
             hbuf, offsets, sorted_slot, T, K, H, I, G, hs, y);
  return hipGetLastError();
}

}  // namespace moe
