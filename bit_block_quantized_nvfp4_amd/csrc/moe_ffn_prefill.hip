// Prefill expert FFN (T > 8 tokens): grouped GEMM on 32x32x16 MFMA, one
// kernel template for both projections.
//
//   gate_up (GU): A = f16 activation rows gathered by token (x with a per-row
//                 power-of-two shift, or the exact f16 value of the FP8 arm's
//                 e4m3 codes), B = NVFP4 gate/up rows dequantised to f16 (one
//                 instruction per element), f32 accumulate; epilogue
//                 h = bf16(silu(g * s2g * f_t) * (u * s2u * f_t)), f_t the
//                 row's epilogue factor.
//   down (DN):    A = bf16 h rows (contiguous sorted positions), B = NVFP4 down
//                 rows dequantised to bf16, epilogue y = bf16(acc * s2d).
//
// Work item = (group, 128-row tile of its sorted rows); the block runs every
// N tile of it in turn.  A block of NW waves owns 64*NW weight rows of an N
// tile: wave w holds two 32-row MFMA blocks (GU: 32 gate rows and the 32 up
// rows of the same pairs; DN: rows 32w and 32*NW + 32w of the tile) against
// all 128 tile rows (four 32-row blocks, the ones past the group's end
// skipped).  Every weight byte is dequantised exactly once per row tile; the
// A tile is shared by all waves.
//
// K runs in steps of 128.  Each step's A tile (the valid 32-row blocks of 128
// rows x 256 B), weight codes (64*NW rows x 64 B) and block scales (64*NW
// rows x 8 B) go from global memory straight into the other half of a
// double-buffered LDS stage by global->LDS DMA, issued one step ahead while
// the current step computes (every 64 B of a weight row by 4 adjacent lanes,
// 16 bytes each); one wait and one barrier per step.  LDS rows are
// XOR-swizzled in 16-byte chunks so that the MFMA operand reads of 16
// consecutive rows at one chunk hit distinct banks.
//
// Lane (n = l%32, q = l/32) of sub-step (c, wd), c in {0,1}, wd in 0..3: MFMA
// k index 8q + i is element 64c + 32q + 8wd + i of the step on both operands
// (weight bytes 32c + 16q + 4wd + i/2 of the row's 64-byte step slice, block
// 4c + 2q + wd/2), so the sums run over all of K.
#include "moe_ffn_common.hpp"
#include "moe_internal.hpp"
#include "moe_prefill_items.hpp"

namespace moe {

// s_waitcnt vmcnt(0) (gfx9 encoding; expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Shared memory of one block (one work item at a time).
template <int NW>
struct PfSmem {
  static constexpr int WR = 64 * NW;
  uint8_t As[2][kPM * 256];  // A tile of a K step, 16-byte chunks swizzled by (row & 15)
  uint8_t Ws[2][WR * 64];    // weight codes of a K step, chunks swizzled by ((row >> 2) & 3)
  uint8_t Ss[2][WR * 8];     // block scales of a K step
  unsigned long long base[kPMaxG];  // item table of pf_find_tile
  unsigned long long wsum[NW];
  int row_src[kPM];          // GU: token of the row; DN: sorted position (valid even for padding)
  float row_fac[kPM];        // GU: epilogue factor of the row's token
  int row_ok[kPM];
};

// The K loop and epilogue of one work item with NMB valid 32-row blocks
// (compile-time, so the MFMA schedule has no branches).
template <int NW, bool GU, int NMB>
__device__ __forceinline__ void pf_item(PfSmem<NW>& sm, const PfTile& ti,
                                        const uint8_t* __restrict__ codes,
                                        const uint8_t* __restrict__ scales,
                                        const float* __restrict__ scale2,
                                        const uint16_t* __restrict__ asrc, int H, int I, int NT,
                                        uint16_t* __restrict__ out) {
  constexpr int NTHR = 64 * NW;
  constexpr int WR = 64 * NW;           // weight rows of a tile
  static_assert(NMB * 32 * 256 % (1024 * NW) == 0, "whole A DMA instructions per wave");
  const int KD = GU ? H : I;  // reduction length
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = ti.g;

  // ---- per-lane DMA sources (fixed across K steps) ----
  // Wave wv moves LDS bytes [1024*(wv + NW*i), +1024) of the A and W stages
  // and [256*(wv + NW*i), +256) of the S stage with one global->LDS DMA
  // instruction each; lane l's bytes land at 16*l (4*l for S), so the lane
  // fetches the global chunk that belongs at that (swizzled) position.
  const size_t rowb = (size_t)KD / 2, srow = (size_t)KD / 16;
  auto wrow = [&](int rho) -> size_t {  // global weight row of tile row rho
    if (GU) {
      const int half = 32 * NW;
      return (size_t)e * 2 * I + (rho < half ? (size_t)ti.nt * half + rho
                                            : (size_t)I + (size_t)ti.nt * half + (rho - half));
    }
    return (size_t)e * H + (size_t)ti.nt * WR + rho;
  };
  // the block runs every N tile of its row tile; N tile j is rows + j * NROWS
  constexpr int NROWS = GU ? 32 * NW : WR;
  const size_t nt_codes = (size_t)NROWS * rowb, nt_scales = (size_t)NROWS * srow;
  constexpr int AI = NMB * 32 * 256 / 1024 / NW;  // A DMA instructions per wave per step (valid row blocks only)
  constexpr int WI = WR * 64 / 1024 / NW;    // = 4 weight DMA instructions
  constexpr int SI = WR * 8 / 256 / NW;      // = 2 scale DMA instructions (4 bytes per lane)
  const uint8_t* asrc_p[AI];
  const uint8_t* wsrc[WI];
  const uint8_t* ssrc[SI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int L = 64 * (wv + NW * i) + lane, r = L >> 4, chp = L & 15;
    asrc_p[i] = (const uint8_t*)(asrc + (size_t)sm.row_src[r] * KD) + 16 * (chp ^ (r & 15));
  }
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int L = 64 * (wv + NW * i) + lane, rho = L >> 2, cpp = L & 3;
    wsrc[i] = codes + wrow(rho) * rowb + 16 * (cpp ^ ((rho >> 2) & 3));
  }
#pragma unroll
  for (int i = 0; i < SI; ++i) {
    const int L = 64 * (wv + NW * i) + lane;
    ssrc[i] = scales + wrow(L >> 1) * srow + 4 * (L & 1);
  }
  int j = 0;  // N tile
  auto dma_step = [&](int jt, int s, int st) {  // N tile jt, K step s, stage st
#pragma unroll
    for (int i = 0; i < AI; ++i)
      __builtin_amdgcn_global_load_lds(asrc_p[i] + 256 * s,
                                       (__attribute__((address_space(3))) void*)&sm.As[st][1024 * (wv + NW * i)],
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < WI; ++i)
      __builtin_amdgcn_global_load_lds(wsrc[i] + jt * nt_codes + 64 * s,
                                       (__attribute__((address_space(3))) void*)&sm.Ws[st][1024 * (wv + NW * i)],
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < SI; ++i)
      __builtin_amdgcn_global_load_lds(ssrc[i] + jt * nt_scales + 8 * s,
                                       (__attribute__((address_space(3))) void*)&sm.Ss[st][256 * (wv + NW * i)],
                                       4, 0, 0);
  };

  const int n32 = lane & 31, q = lane >> 5;
  int rho_b[2];
  rho_b[0] = 32 * wv + n32;
  rho_b[1] = 32 * NW + 32 * wv + n32;

  for (; j < NT; ++j) {
    f32x16 acc[NMB][2];
  #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
  #pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{};

    const int nsteps = KD / kPK;
    if (j == 0) {  // later tiles had their first step prefetched by the previous tile
      dma_step(0, 0, 0);
      wait_vmcnt0();
      __syncthreads();
    }
    for (int s = 0; s < nsteps; ++s) {
      const int st = (j * nsteps + s) & 1;  // stage parity runs on across N tiles
      // stage st ^ 1 was last read in step s - 1, which every wave has finished
      if (s + 1 < nsteps) dma_step(j, s + 1, st ^ 1);
      else if (j + 1 < NT) dma_step(j + 1, 0, st ^ 1);  // the next tile's first step
      const uint8_t* A = sm.As[st];
      const uint8_t* Wt = sm.Ws[st];
      const uint8_t* St = sm.Ss[st];
      u32x2 sw[2];
      u32x4 wc[2][2];
  #pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int rho = rho_b[nb];
        sw[nb] = *(const u32x2*)(St + rho * 8);
  #pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int cp = 2 * c + q;
          wc[c][nb] = *(const u32x4*)(Wt + rho * 64 + 16 * (cp ^ ((rho >> 2) & 3)));
        }
      }
      // this lane's two block scales of chunk c: bytes 4c + 2q, 4c + 2q + 1
      uint32_t sp[2][2];
  #pragma unroll
      for (int c = 0; c < 2; ++c)
  #pragma unroll
        for (int nb = 0; nb < 2; ++nb) sp[c][nb] = q ? (sw[nb][c] >> 16) : sw[nb][c];
      // the A operands of sub-step t = 4c + wd are read one sub-step ahead
      auto read_a = [&](int t, u32x4 (&av)[NMB]) {
        const int ach = 8 * (t >> 2) + 4 * q + (t & 3);
  #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const int r = 32 * mb + n32;
          av[mb] = *(const u32x4*)(A + r * 256 + 16 * (ach ^ (r & 15)));
        }
      };
      u32x4 av_cur[NMB], av_nxt[NMB];
      read_a(0, av_cur);
  #pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int c = t >> 2, wd = t & 3;
        if (t < 7) read_a(t + 1, av_nxt);
        u32x4 b[2];
  #pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if (GU) {
            const f16x2 sv = e4m3x2_to_f16(sp[c][nb]);
            b[nb] = __builtin_bit_cast(u32x4, dqh8(wc[c][nb][wd], wd < 2 ? sv.x : sv.y));
          } else {
            const f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sp[c][nb], 1.0f, false);
            b[nb] = __builtin_bit_cast(u32x4, dq8(wc[c][nb][wd], wd < 2 ? sv.x : sv.y));
          }
        }
  #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
  #pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            if (GU)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  as_f16x8(av_cur[mb]), as_f16x8(b[nb]), acc[mb][nb], 0, 0, 0);
            else
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  as_bf16x8(av_cur[mb]), as_bf16x8(b[nb]), acc[mb][nb], 0, 0, 0);
          }
        }
        if (t < 7) {
  #pragma unroll
          for (int mb = 0; mb < NMB; ++mb) av_cur[mb] = av_nxt[mb];
        }
      }
      wait_vmcnt0();     // this wave's DMA of the next step has landed
      __syncthreads();   // ... and every wave's; stage st is free again
    }

    // ---- epilogue ----
    // opaque copies (p0, and a zero added to the row-table offsets): the
    // epilogue's addresses and row flags are rebuilt for each N tile instead
    // of being hoisted out of the N-tile loop into registers
    int p0 = ti.p0, z = 0;
    asm volatile("" : "+s"(p0), "+s"(z));
    if (GU) {
      const float s2g = scale2[3 * e + 0], s2u = scale2[3 * e + 1];
      const int col = j * 32 * NW + 32 * wv + n32;
  #pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
  #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * mb + 8 * (i >> 2) + 4 * q + (i & 3);
          if (r < ti.rows && sm.row_ok[r + z]) {
            const float f = sm.row_fac[r + z];
            const float g = acc[mb][0][i] * s2g * f, u = acc[mb][1][i] * s2u * f;
            out[(size_t)(p0 + r) * I + col] = f32_to_bf16_bits(silu_f32(g) * u);
          }
        }
      }
    } else {
      const float s2d = scale2[3 * e + 2];
  #pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
  #pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = j * WR + 32 * NW * nb + 32 * wv + n32;
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 32 * mb + 8 * (i >> 2) + 4 * q + (i & 3);
            if (r < ti.rows && sm.row_ok[r + z])
              out[(size_t)(p0 + r) * H + col] = f32_to_bf16_bits(acc[mb][nb][i] * s2d);
          }
        }
      }
    }
  }
}

template <int NW, bool GU>
__global__ __launch_bounds__(64 * NW, 1) void k_prefill_gemm(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ scale2, const uint16_t* __restrict__ asrc,
    const float* __restrict__ rowfac, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slot, int T, int K, int H, int I, int G, int has_shared,
    int shared_rows, uint16_t* __restrict__ out) {
  constexpr int NTHR = 64 * NW;
  __shared__ __align__(16) PfSmem<NW> sm;
  const int NT = GU ? I / (32 * NW) : H / (64 * NW);  // N tiles per group
  PfTile ti;
  if (!pf_find_tile<NTHR>(offsets, G, 1, sm.base, sm.wsum, &ti)) return;  // item = row tile
  const int tid = threadIdx.x;
  // gate_up: the shared group reads activation rows shared_rows + t (its own arm)
  const int roff = (GU && has_shared && ti.g == G - 1) ? shared_rows : 0;
  for (int r = tid; r < kPM; r += NTHR) {
    int src = -1;
    if (r < ti.rows) {
      const int tk = slot_token(sorted_slot[ti.p0 + r], T, K, has_shared);
      src = tk < 0 ? -1 : (GU ? tk + roff : ti.p0 + r);
    }
    sm.row_ok[r] = src >= 0;
    sm.row_src[r] = src >= 0 ? src : (GU ? 0 : ti.p0);  // a valid row to read for padding rows
    if (GU) sm.row_fac[r] = src >= 0 ? rowfac[src] : 0.f;
  }
  __syncthreads();
  switch ((ti.rows + 31) / 32) {  // uniform per block
    case 1: pf_item<NW, GU, 1>(sm, ti, codes, scales, scale2, asrc, H, I, NT, out); break;
    case 2: pf_item<NW, GU, 2>(sm, ti, codes, scales, scale2, asrc, H, I, NT, out); break;
    case 3: pf_item<NW, GU, 3>(sm, ti, codes, scales, scale2, asrc, H, I, NT, out); break;
    default: pf_item<NW, GU, 4>(sm, ti, codes, scales, scale2, asrc, H, I, NT, out); break;
  }
}

void register_prefill_kernels(std::vector<const void*>& k) {
  k.push_back((const void*)&k_prefill_gemm<8, true>);
  k.push_back((const void*)&k_prefill_gemm<4, true>);
  k.push_back((const void*)&k_prefill_gemm<8, false>);
  k.push_back((const void*)&k_prefill_gemm<4, false>);
}

hipError_t launch_prefill_ffn(const moe_nvfp4_weights& W, int T, int K, const int32_t* offsets,
                              const int32_t* sorted_slot, const _Float16* xh, const float* rowfac,
                              int shared_rows, uint16_t* hbuf, uint16_t* y, hipStream_t s) {
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const int G = W.E + hs;
  const long S = (long)T * K + (hs ? T : 0);
  // at most S/kPM full row tiles plus one partial tile per group
  const long mt_bound = S / kPM + G;
  const uint16_t* xa = (const uint16_t*)xh;
  if (I % 256 == 0) {
    const dim3 g1((unsigned)mt_bound);
    MOE_LAUNCH("grouped_gate_up", s, (k_prefill_gemm<8, true>), g1, dim3(512), 0, s, W.gu_codes,
               W.gu_scales, W.scale2, xa, rowfac, offsets, sorted_slot, T, K, H, I, G, hs, shared_rows, hbuf);
  } else {
    const dim3 g1((unsigned)mt_bound);
    MOE_LAUNCH("grouped_gate_up", s, (k_prefill_gemm<4, true>), g1, dim3(256), 0, s, W.gu_codes,
               W.gu_scales, W.scale2, xa, rowfac, offsets, sorted_slot, T, K, H, I, G, hs, shared_rows, hbuf);
  }
  if (H % 512 == 0) {
    const dim3 g2((unsigned)mt_bound);
    MOE_LAUNCH("grouped_down", s, (k_prefill_gemm<8, false>), g2, dim3(512), 0, s, W.dn_codes,
               W.dn_scales, W.scale2, hbuf, nullptr, offsets, sorted_slot, T, K, H, I, G, hs, 0, y);
  } else {
    const dim3 g2((unsigned)mt_bound);
    MOE_LAUNCH("grouped_down", s, (k_prefill_gemm<4, false>), g2, dim3(256), 0, s, W.dn_codes,
               W.dn_scales, W.scale2, hbuf, nullptr, offsets, sorted_slot, T, K, H, I, G, hs, 0, y);
  }
  return hipGetLastError();
}

}  // namespace moe
