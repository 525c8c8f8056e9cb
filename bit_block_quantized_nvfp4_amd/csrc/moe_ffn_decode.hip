// Decode/verify expert FFN (T <= 8 tokens): a multi-row GEMV on MFMA that
// streams each active expert's NVFP4 weights once (gate+up fused with SiLU,
// then down; routed experts and the shared expert in the same launches).
//
// The work is memory-bound: one wave is one work unit and covers the whole K
// of its rows.  The unit's activation (or h) rows and block scales are issued
// first, then its code chunks in a short software pipeline, fully unrolled
// (no loop back edge, so the waits are exact vmcnt counts): a couple of
// chunks ahead of the one the MFMAs consume.  Issuing every chunk up front
// fills the memory pipeline at once, the issue then stalls, and each wave's
// activation rows and first MFMA come late in the stream; with the pipeline
// the rows land first and the dequant/MFMA work spreads over the stream.
// Many resident waves per CU keep HBM busy; a block holds 1 wave when the
// units would not fill the chip and 4 (one LDS copy of the activations) when
// they would.
//
// k_dec_xprep (the grouped-GEMM path's activation prep, one block per token
// row): each row of x becomes f16 with a power-of-two shift (bf16 arm; the
// shift is undone in the f32 epilogue, see f16_row_shift) or, for the FP8 arm,
// is quantised to e4m3 per row and kept as the (exact) f16 value of each code,
// with the row scale as epilogue factor.  The decode path applies the same
// rule inside k_dec_gate_up, on the rows it has staged in LDS.
//
// k_dec_gate_up: unit = (active group, 16 gate/up row pairs).  The MFMA runs
// over the rows of ALL T tokens (T <= 8 of its 16 rows) and the epilogue keeps
// the tokens routed to the group, so the activation rows go to LDS before the
// group is even known.  f16 MFMA 16x16x32; weights are dequantised to f16
// exactly with one instruction per element.
//
// k_dec_down: unit = (active group, 16 NB output rows as NB MFMA blocks of
// 16; NB = 4, or fewer when the units would not fill the chip);
// A = the group's h rows (bf16, by sorted position), up to 16 per pass, in
// LDS, turned into f16 in place with a per-row power-of-two shift (undone in
// the epilogue); f16 MFMA 16x16x32 against weights dequantised to f16 at one
// instruction per element.
//
// Lane (r = l%16, q = l/16) of either kernel: B column r = weight row, A row r
// = token row (or group row).  The lane's 16-byte code chunk c is bytes
// [64c + 16q, +16) of its weight row, i.e. elements 128c + 32q + [0, 32), and
// 32-bit word j of it feeds sub-MFMA (c, j): MFMA k index 8q + i maps to
// element 128c + 32q + 8j + i on both operands, so the sum is over all of K.
#include <type_traits>

#include "moe_combine.hpp"
#include "moe_ffn_common.hpp"
#include "moe_internal.hpp"
#include "moe_route_permute.hpp"
#include "moe_xprep.hpp"

namespace moe {

// ------------------------------- x prep ------------------------------------

template <bool FP8>
__global__ __launch_bounds__(256) void k_dec_xprep(const uint16_t* __restrict__ x, int H,
                                                   _Float16* __restrict__ xh,
                                                   float* __restrict__ unmul,
                                                   uint8_t* __restrict__ xq,
                                                   float* __restrict__ xs) {
  __shared__ float wmax[4];
  xprep_row<FP8>(x, H, blockIdx.x, xh, unmul, xq, xs, wmax);
}

// ------------------------------- gate_up ----------------------------------
// One wave = one unit (group, 16 gate/up row pairs, all of K); a block holds
// WPB waves = WPB consecutive units of one group and one LDS copy of the f16
// activation rows.
//
// Code loads are row-contiguous: lane (r16, q) reads bytes [64c + 16q, +16)
// of weight row r16 for c = 0 .. NCH-1, so every load instruction covers 64
// contiguous bytes of each of 16 rows (measured on the device: 4.5 TB/s for
// this pattern against 2.7 TB/s when each lane's 16 bytes sit in a segment of
// their own).  Word j of chunk c holds elements 128c + 32q + 8j + [0, 8),
// block 8c + 2q + j/2.  The block scales of the unit's rows are two
// contiguous runs (16 gate rows, 16 up rows, H/16 bytes each) and go to LDS
// by DMA; each chunk's scale pair is read from there.
//
// Load order (all issued before the first wait): the activation rows straight
// into LDS (global->LDS DMA, no registers; they do not depend on the group),
// the group lookup, the unit's scale runs into LDS, every code word of the
// unit, then the epilogue's metadata.  The activation rows are unpadded with
// the 16-byte chunk index XOR-swizzled by (row & 15), so the A-operand reads
// of 16 rows at one chunk hit 16 distinct bank groups.

// Copy BYTES contiguous bytes (a multiple of 256) from global memory to LDS
// with one wave: 16 bytes per lane when BYTES is a multiple of 1 KB, else 4.
template <int BYTES>
__device__ __forceinline__ void dma_run(const uint8_t* g, uint8_t* lds, int lane) {
  static_assert(BYTES % 256 == 0, "whole DMA instructions");
  if constexpr (BYTES % 1024 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 1024; ++i) dma16(g + 1024 * i + 16 * lane, lds + 1024 * i);
  } else {
#pragma unroll
    for (int i = 0; i < BYTES / 256; ++i)
      __builtin_amdgcn_global_load_lds(g + 256 * i + 4 * lane,
                                       (__attribute__((address_space(3))) void*)(lds + 256 * i), 4,
                                       0, 0);
  }
}

// Copy rows [0, nrows) of a row-major matrix of 16-bit values (row length
// cpr 16-byte chunks, cpr >= 16) into LDS, chunk ch of row r stored at chunk
// position r*cpr + (ch ^ (r & 15)).  Source row r is src_row(r).  Wave wv of
// nw moves LDS chunks [64*(wv + nw*i), +64) with one DMA instruction each.
template <typename RowPtr>
__device__ __forceinline__ void dma_rows_swizzled(void* lds, int nrows, int cpr, int wv, int nw,
                                                  int lane, RowPtr src_row) {
  const int total = nrows * cpr;
  for (int base = 64 * wv; base < total; base += 64 * nw) {
    const int L = base + lane;
    if (L < total) {
      const int r = L / cpr, ch = (L % cpr) ^ (r & 15);
      dma16(src_row(r) + 16 * ch, (uint8_t*)lds + 16 * base);
    }
  }
}

// Byte offset in such an LDS copy of chunk ch of row r.
__device__ __forceinline__ int swz_off(int r, int ch, int cpr) {
  return 16 * (r * cpr + (ch ^ (r & 15)));
}

// s_waitcnt limiting only the vector-memory counter to N (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14]; expcnt [6:4] and lgkmcnt [11:8] at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// Code chunks of a unit in flight ahead of the one being consumed (gate_up,
// down); measured at H = 2048, I = 512, T = 8: gate_up 26.6 us with every
// chunk issued up front, 24.7 / 22.6 / 21.9 / 21.1 us with 8 / 4 / 3 / 2
// ahead; down 14.9 us before, 13.5 - 13.8 us with 1, 2 or 4 ahead (the gain
// there is the h rows issued ahead of the weights).
constexpr int kGuPipe = 2;
constexpr int kDnPipe = 2;

// Activation rows -> f16 MFMA operand in LDS, in place (the rule of
// k_dec_xprep, bit for bit): wave wv of WPB converts rows wv, wv + WPB, ...
// of the TR staged rows (chunk-swizzled, CPR 16-byte chunks per row); the
// row's epilogue factor goes to fac[]; with fp8_row, the row is quantised to
// e4m3 (and with write_q its codes and scale go to xq / xs).
template <int CPR, int TR, int WPB>
__device__ __forceinline__ void dec_convert_rows(_Float16* xl, float* fac, float* __restrict__ xs,
                                                 uint8_t* __restrict__ xq, int H, int T,
                                                 bool fp8_row, bool write_q, int wv, int lane) {
  constexpr int NCL = (CPR + 63) / 64;  // chunks of a row per lane
  for (int r = wv; r < TR; r += WPB) {
    float amax = 0.f;
    {
      u32x4 v[NCL];
#pragma unroll
      for (int k = 0; k < NCL; ++k) {
        const int ch = lane + 64 * k;
        v[k] = ch < CPR ? *(const u32x4*)((const uint8_t*)xl + swz_off(r, ch, CPR))
                        : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int k = 0; k < NCL; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[k][j] & 0xFFFFu)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[k][j] >> 16)));
        }
    }
    amax = wave_max_nonneg(amax);  // fmaxf drops NaN: every lane is >= 0, not NaN
    float mul, rf;
    if (fp8_row) {
      rf = amax > 0.f ? amax / 448.0f : 1.0f;
      mul = amax > 0.f ? 448.0f / amax : 1.0f;
    } else {
      const int sh = f16_row_shift(amax);
      mul = ldexpf(1.0f, sh);
      rf = ldexpf(1.0f, -sh);
    }
    const bool wr = write_q && fp8_row && r < T;
    if (lane == 0) {
      fac[r] = rf;
      if (wr) xs[r] = rf;
    }
    u32x4 vr[NCL];
#pragma unroll
    for (int k = 0; k < NCL; ++k) {
      const int ch = lane + 64 * k;
      vr[k] = ch < CPR ? *(const u32x4*)((const uint8_t*)xl + swz_off(r, ch, CPR))
                       : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < NCL; ++k) {
      const int ch = lane + 64 * k;
      if (ch >= CPR) break;
      uint8_t* pch = (uint8_t*)xl + swz_off(r, ch, CPR);
      const u32x4 v = vr[k];
      u32x4 o;
      if (fp8_row) {
        u32x2 code;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float f0 = bf16_bits_to_f32(v[2 * j] & 0xFFFFu) * mul;
          float f1 = bf16_bits_to_f32(v[2 * j] >> 16) * mul;
          float f2 = bf16_bits_to_f32(v[2 * j + 1] & 0xFFFFu) * mul;
          float f3 = bf16_bits_to_f32(v[2 * j + 1] >> 16) * mul;
          f0 = fminf(fmaxf(f0, -448.f), 448.f);
          f1 = fminf(fmaxf(f1, -448.f), 448.f);
          f2 = fminf(fmaxf(f2, -448.f), 448.f);
          f3 = fminf(fmaxf(f3, -448.f), 448.f);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, w, true);
          code[j] = (uint32_t)w;
        }
        if (wr) *(u32x2*)(xq + (size_t)r * H + 8 * ch) = code;
        const u32x2 lo = fp8x4_to_f16(code.x), hi = fp8x4_to_f16(code.y);
        o = u32x4{lo.x, lo.y, hi.x, hi.y};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = pack_f16x2(bf16_bits_to_f32(v[j] & 0xFFFFu) * mul,
                            bf16_bits_to_f32(v[j] >> 16) * mul);
      }
      *(u32x4*)pch = o;
    }
  }
}

// TR = activation rows staged (T rounded up to 1, 2, 4 or 8; rows >= T repeat
// row T-1), which makes the number of DMA instructions per wave a constant.
// Dynamic LDS: [TR][H] activation rows (bf16 as loaded, f16 after the in-place
// conversion), 8 row factors, then per wave the gate and up scale runs
// (2 x 16 x H/16 bytes).
//
// KS > 1 (split K, for launches whose units would not fill the chip): a block
// is ONE unit and its KS = WPB waves take NCH / KS consecutive chunks each, so
// every unit has KS waves' loads in flight instead of one.  The block's scale
// runs are one LDS copy, each wave moving an equal piece of it; each wave's
// partial sums go to LDS and wave 0 adds them in wave order (a fixed order:
// the result does not depend on timing) before the epilogue.  LDS then holds
// one pair of scale runs and (KS - 1) x 512 floats of partial sums.
//
// The activation rows are turned into the f16 MFMA operand in LDS, in place,
// by the block itself (the rule of k_dec_xprep, bit for bit): wave wv converts
// rows wv, wv + WPB, ...; the row's epilogue factor goes to LDS.  With FP8,
// block 0 also writes the row codes and scales to xq / xs.
template <int NCH, int WPB, int TR, bool FP8, int KS>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(3))) void k_dec_gate_up(
    const uint8_t* __restrict__ gu_codes, const uint8_t* __restrict__ gu_scales,
    const float* __restrict__ scale2, const uint16_t* __restrict__ x,
    uint8_t* __restrict__ xq, float* __restrict__ xs, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slot, const int32_t* __restrict__ groups, int T, int K,
    int H, int I, int has_shared, int fp8_sel, int shared_g, uint16_t* __restrict__ h) {
  extern __shared__ __align__(16) _Float16 xl[];
  constexpr int CPR = 16 * NCH;                     // 16-byte chunks per row, H = 128 * NCH
  constexpr int NDMA = (TR * CPR + 64 * WPB - 1) / (64 * WPB);
  constexpr int SRUN = 128 * NCH;                   // scale bytes of 16 rows
  static_assert(KS == 1 || (KS == WPB && NCH % KS == 0 && KS % 2 == 0),
                "split K: one unit per block, whole chunks per wave, whole scale runs per wave pair");
  constexpr int NCK = NCH / KS;                     // chunks per wave
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, r16 = lane & 15, q = lane >> 4;
  const int nbk = KS > 1 ? I / 16 : I / 16 / WPB;
  const int a = blockIdx.x / nbk;
  const int pb = KS > 1 ? blockIdx.x % nbk : (blockIdx.x % nbk) * WPB + wv;
  const int c0 = KS > 1 ? wv * NCK : 0;             // this wave's first chunk

  // (1) activation rows (bf16) -> LDS, first of all: they do not depend on
  // the group, and issued ahead of every code load on the CU they land early,
  // so their conversion stays off the critical path
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int base = 64 * (wv + WPB * i), L = base + lane;
    if (L < TR * CPR) {
      const int r = L / CPR, ch = (L % CPR) ^ (r & 15);
      dma16(x + (size_t)(r < T ? r : T - 1) * H + 8 * ch, (uint8_t*)xl + 16 * base);
    }
  }
  float* fac = (float*)((uint8_t*)xl + (size_t)TR * H * 2);
  // Activation rows -> f16 MFMA operand in LDS, in place (the rule of
  // k_dec_xprep, bit for bit): wave wv converts rows wv, wv + WPB, ...; the
  // row's epilogue factor goes to fac[]; with FP8, block 0 also writes the
  // row codes and scales to xq / xs.
  auto convert_rows = [&](bool fp8_row) {
    dec_convert_rows<CPR, TR, WPB>(xl, fac, xs, xq, H, T, fp8_row, fp8_sel == 0 && blockIdx.x == 0,
                                   wv, lane);
  };
  // a < min(T*K + S, E') <= E', so groups[1 + a] is in bounds; both words in one trip
  const int nact = groups[0], e = groups[1 + a];
  asm volatile("" ::"s"(e));  // (keeps the second lookup above the branch)
  if (a >= nact) {            // uniform per block: nothing to do, but the DMA into
    wait_vmcnt<0>();          // this block's LDS must land before the block ends
    if (FP8 && fp8_sel == 0 && blockIdx.x == 0) {  // the row codes and scales are outputs
      __builtin_amdgcn_s_barrier();  // of the call even when no group is active
      convert_rows(true);
    }
    return;
  }
  uint8_t* sl = (uint8_t*)xl + (size_t)TR * H * 2 + 256 + (KS > 1 ? 0 : (size_t)wv * 2 * SRUN);

  // the unit's scale runs -> LDS (with split K, wave wv moves bytes
  // [wv P, (wv + 1) P) of the gate run followed by the up run)
  const size_t grow = (size_t)e * 2 * I + (size_t)pb * 16;  // first gate row of the unit
  constexpr int SPIECE = KS > 1 ? 2 * SRUN / KS : SRUN;
  {
    const uint8_t* sg = gu_scales + grow * (H / 16);
    if constexpr (KS == 1) {
      dma_run<SRUN>(sg, sl, lane);
      dma_run<SRUN>(sg + (size_t)I * (H / 16), sl + SRUN, lane);
    } else {
      const int off = wv * SPIECE;
      dma_run<SPIECE>(off < SRUN ? sg + off : sg + (size_t)I * (H / 16) + (off - SRUN), sl + off,
                      lane);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);  // nothing below moves above the DMA

  // (2) the epilogue's metadata; the slot of position `lane` is loaded for
  // every lane (clamped into the group, n >= 1)
  const int p0 = offsets[e], n = offsets[e + 1] - p0;
  const float s2g = scale2[3 * e + 0], s2u = scale2[3 * e + 1];
  const int slot_l = sorted_slot[p0 + (lane < n ? lane : n - 1)];
  __builtin_amdgcn_sched_barrier(0);  // the slot load stays ahead of the code loads

  // (3) the code words of the unit, 2 row-contiguous 16-byte loads per chunk
  // of 128 K, software-pipelined: the first kGuPipe chunks now, then chunk
  // c + kGuPipe right after chunk c is consumed.  Every wave then computes
  // while its later chunks stream in, instead of issuing all of them first
  // (the issue stalls once the memory pipeline is full, which delayed every
  // wave's first MFMA to late in the stream).
  constexpr int D = NCK < kGuPipe ? NCK : kGuPipe;
  const size_t rowb = (size_t)H / 2;
  const uint8_t* cg = gu_codes + (grow + r16) * rowb + 16 * q + 64 * c0;
  const uint8_t* cu = cg + (size_t)I * rowb;
  u32x4 wg[NCK], wu[NCK];
  auto issue = [&](int c) {
    wg[c] = *(const u32x4*)(cg + 64 * c);
    wu[c] = *(const u32x4*)(cu + 64 * c);
  };
#pragma unroll
  for (int c = 0; c < D; ++c) issue(c);
  __builtin_amdgcn_sched_barrier(0);

  // (4) this wave's activation DMA is complete once at most the scale DMA,
  // the slot load and the first code loads are outstanding; the barrier
  // then covers the whole block.
  constexpr int kScaleDma = (KS > 1 ? 1 : 2) * (SPIECE % 1024 == 0 ? SPIECE / 1024 : SPIECE / 256);
  wait_vmcnt<kScaleDma + 1 + 2 * D>();
  __builtin_amdgcn_s_barrier();

  // (5) activation rows -> f16 in place (LDS only).  Two passes over each row
  // in LDS (absmax, then convert), one row at a time; each pass issues all of
  // the lane's chunks of the row at once, and the absmax reduction is DPP-only.
  // the arm of this block's group: every group (fp8_sel 0), only the routed
  // groups (1) or only the shared group (2) read e4m3 rows
  const bool shared_grp = e == shared_g;  // shared_g = E with a shared expert, else -1
  convert_rows(FP8 && (fp8_sel == 0 || (fp8_sel == 1) != shared_grp));
  // the scale runs and the slot have landed once only the code loads are
  // outstanding; LDS traffic done, then the barrier publishes the rows.
  wait_vmcnt<2 * D>();
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  float ums[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) ums[t] = fac[t < TR ? t : TR - 1];

  // A row r16 of the MFMA = token r16; rows >= T read row T-1 (never stored)
  const int xr = r16 < T ? r16 : T - 1;
  const uint8_t* xrow = (const uint8_t*)xl;
  const uint8_t* srow = sl + r16 * (8 * NCH) + 2 * q + 8 * c0;
  // the swizzle touches only the low 4 bits of the chunk index, so the
  // operand of sub-MFMA (c, j) sits at aoff[j] + 256 c (an immediate offset)
  int aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aoff[j] = swz_off(xr, 4 * q + j, CPR) + 256 * c0;
  f32x4 dg = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
  static_for<0, NCK>([&](auto ct) {
    constexpr int c = decltype(ct)::value;
    // chunks issued so far: min(NCK, D + c); chunk c is complete once the
    // ones after it are the only loads outstanding
    constexpr int issued = D + c < NCK ? D + c : NCK;
    wait_vmcnt<2 * (issued - c - 1)>();
    const f16x2 sgv = e4m3x2_to_f16(*(const uint16_t*)(srow + 8 * c));
    const f16x2 suv = e4m3x2_to_f16(*(const uint16_t*)(srow + SRUN + 8 * c));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x8 av = *(const f16x8*)(xrow + aoff[j] + 256 * c);
      dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(wg[c][j], j < 2 ? sgv.x : sgv.y), dg, 0, 0, 0);
      du = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(wu[c][j], j < 2 ? suv.x : suv.y), du, 0, 0, 0);
    }
    if constexpr (c + D < NCK) issue(c + D);
    __builtin_amdgcn_sched_barrier(0);
  });
  if constexpr (KS > 1) {
    // partial sums of waves 1 .. KS-1 -> LDS ([wave][8][64] floats, lane
    // fastest); wave 0 adds them in wave order and runs the epilogue alone
    float* red = (float*)(sl + 2 * SRUN);
    if (wv > 0) {
      float* dst = red + (size_t)(wv - 1) * 512 + lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[64 * i] = dg[i];
        dst[64 * (4 + i)] = du[i];
      }
    }
    __syncthreads();
    if (wv > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dg[i] += red[512 * w + 64 * i + lane];
        du[i] += red[512 * w + 64 * (4 + i) + lane];
      }
  }
  uint16_t hv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float um = q == 0 ? ums[i] : (q == 1 ? ums[4 + i] : 0.f);  // tokens >= 8 are never stored
    const float g = dg[i] * um * s2g, u = du[i] * um * s2u;
    hv[i] = f32_to_bf16_bits(silu_f32(g) * u);
  }
  // position p of the group holds token tok(p); lane (tok/4, col) has its row
  const int tokl = slot_token(slot_l, T, K, has_shared);
  const int j = pb * 16 + r16;
  for (int p = 0; p < n; ++p) {
    const int tok = p < 64 ? __shfl(tokl, p, 64) : slot_token(sorted_slot[p0 + p], T, K, has_shared);
    if (tok >= 0 && (tok >> 2) == q) {
      const int i = tok & 3;
      h[(size_t)(p0 + p) * I + j] = i == 0 ? hv[0] : (i == 1 ? hv[1] : (i == 2 ? hv[2] : hv[3]));
    }
  }
}

// Whole-CU gate_up: one block of kGuCuWaves waves per CU stages and converts
// the activation rows once and takes an equal share (within one unit) of the
// launch's active units, split at run time from the active group count; wave
// w takes units u0 + w, u0 + w + kGuCuWaves, ... of its block's share.  Each
// CU then streams the same amount of weights: with blocks of 4 units, 2.5
// blocks per CU on average leave some CUs with 3 blocks and others with 2,
// and the kernel waits for the CUs with 3 (measured at T=8: 18.0 us against
// 13.4 us).  The unit itself is k_dec_gate_up's (same loads, pipeline, MFMAs
// and epilogue, so the same bits).  All units of a block read one activation
// form, so the per-class FP8 arms keep k_dec_gate_up.
constexpr int kGuCuWaves = 16;
// LDS bytes per wave of the decode layer kernel: the unit's two scale runs
// (16 rows x H/16 bytes each) and, with split K, at least the partial sums of
// the wave's 16 x 32 outputs (2 KB).
constexpr int dec_layer_slot_bytes(int nch, int ks) {
  return ks > 1 && 256 * nch < 2048 ? 2048 : 256 * nch;
}

template <int NCH, int TR, bool FP8>
__global__ __launch_bounds__(64 * kGuCuWaves) void k_dec_gate_up_cu(
    const uint8_t* __restrict__ gu_codes, const uint8_t* __restrict__ gu_scales,
    const float* __restrict__ scale2, const uint16_t* __restrict__ x,
    uint8_t* __restrict__ xq, float* __restrict__ xs, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slot, const int32_t* __restrict__ groups, int T, int K,
    int H, int I, int has_shared, uint16_t* __restrict__ h) {
  constexpr int WPB = kGuCuWaves;
  extern __shared__ __align__(16) _Float16 xl[];
  constexpr int CPR = 16 * NCH;                     // 16-byte chunks per row, H = 128 * NCH
  constexpr int NDMA = (TR * CPR + 64 * WPB - 1) / (64 * WPB);
  constexpr int SRUN = 128 * NCH;                   // scale bytes of 16 rows
  constexpr int D = NCH < kGuPipe ? NCH : kGuPipe;
  constexpr int kScaleDma = 2 * (SRUN % 1024 == 0 ? SRUN / 1024 : SRUN / 256);
  const int lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // (1) activation rows (bf16) -> LDS, first of all (every wave)
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int base = 64 * (wv + WPB * i), L = base + lane;
    if (L < TR * CPR) {
      const int r = L / CPR, ch = (L % CPR) ^ (r & 15);
      dma16(x + (size_t)(r < T ? r : T - 1) * H + 8 * ch, (uint8_t*)xl + 16 * base);
    }
  }
  float* fac = (float*)((uint8_t*)xl + (size_t)TR * H * 2);
  uint8_t* sl = (uint8_t*)xl + (size_t)TR * H * 2 + 256 + (size_t)wv * 2 * SRUN;

  // (2) this block's share of the active units
  const int nbk = I / 16;
  const int units = groups[0] * nbk;
  const int u0 = (int)((long long)blockIdx.x * units / gridDim.x);
  const int u1 = (int)((long long)(blockIdx.x + 1) * units / gridDim.x);

  // per-unit state: the unit's group, metadata, code pointers and words
  const size_t rowb = (size_t)H / 2;
  int e = 0, pb = 0, p0 = 0, n = 1, slot_l = 0;
  float s2g = 0.f, s2u = 0.f;
  const uint8_t* cg = gu_codes;
  const uint8_t* cu = gu_codes;
  u32x4 wg[NCH], wu[NCH];
  auto issue = [&](int c) {
    wg[c] = *(const u32x4*)(cg + 64 * c);
    wu[c] = *(const u32x4*)(cu + 64 * c);
  };
  // the unit's scale runs (DMA), its metadata and slot, and its first D code
  // chunks, in that order
  auto begin_unit = [&](int uu) {
    const int a = uu / nbk;
    pb = uu % nbk;
    e = groups[1 + a];
    const size_t grow = (size_t)e * 2 * I + (size_t)pb * 16;  // first gate row of the unit
    const uint8_t* sg = gu_scales + grow * (H / 16);
    dma_run<SRUN>(sg, sl, lane);
    dma_run<SRUN>(sg + (size_t)I * (H / 16), sl + SRUN, lane);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    p0 = offsets[e];
    n = offsets[e + 1] - p0;
    s2g = scale2[3 * e + 0];
    s2u = scale2[3 * e + 1];
    slot_l = sorted_slot[p0 + (lane < n ? lane : n - 1)];
    __builtin_amdgcn_sched_barrier(0);
    cg = gu_codes + (grow + r16) * rowb + 16 * q;
    cu = cg + (size_t)I * rowb;
#pragma unroll
    for (int c = 0; c < D; ++c) issue(c);
    __builtin_amdgcn_sched_barrier(0);
  };
  const bool has = u0 + wv < u1;  // uniform per wave
  if (has) begin_unit(u0 + wv);
  // this wave's activation DMA is complete once at most its scale DMA, slot
  // load and first code loads are outstanding; the barrier covers the block
  if (has) wait_vmcnt<kScaleDma + 1 + 2 * D>();
  else wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  dec_convert_rows<CPR, TR, WPB>(xl, fac, xs, xq, H, T, FP8, FP8 && blockIdx.x == 0, wv, lane);
  if (has) wait_vmcnt<2 * D>();  // the scale runs and the slot have landed
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  if (!has) return;

  float ums[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) ums[t] = fac[t < TR ? t : TR - 1];
  const int xr = r16 < T ? r16 : T - 1;
  const uint8_t* xrow = (const uint8_t*)xl;
  const uint8_t* srow = sl + r16 * (8 * NCH) + 2 * q;
  int aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aoff[j] = swz_off(xr, 4 * q + j, CPR);
  // the MFMAs of the unit (chunk c once it has landed, then chunk c + D is
  // issued) and its epilogue
  auto compute_unit = [&]() {
    f32x4 dg = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
    static_for<0, NCH>([&](auto ct) {
      constexpr int c = decltype(ct)::value;
      constexpr int issued = D + c < NCH ? D + c : NCH;
      wait_vmcnt<2 * (issued - c - 1)>();
      const f16x2 sgv = e4m3x2_to_f16(*(const uint16_t*)(srow + 8 * c));
      const f16x2 suv = e4m3x2_to_f16(*(const uint16_t*)(srow + SRUN + 8 * c));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x8 av = *(const f16x8*)(xrow + aoff[j] + 256 * c);
        dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(wg[c][j], j < 2 ? sgv.x : sgv.y), dg, 0, 0, 0);
        du = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(wu[c][j], j < 2 ? suv.x : suv.y), du, 0, 0, 0);
      }
      if constexpr (c + D < NCH) issue(c + D);
      __builtin_amdgcn_sched_barrier(0);
    });
    uint16_t hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float um = q == 0 ? ums[i] : (q == 1 ? ums[4 + i] : 0.f);  // tokens >= 8 are never stored
      const float g = dg[i] * um * s2g, u = du[i] * um * s2u;
      hv[i] = f32_to_bf16_bits(silu_f32(g) * u);
    }
    const int tokl = slot_token(slot_l, T, K, has_shared);
    const int j = pb * 16 + r16;
    for (int p = 0; p < n; ++p) {
      const int tok = p < 64 ? __shfl(tokl, p, 64) : slot_token(sorted_slot[p0 + p], T, K, has_shared);
      if (tok >= 0 && (tok >> 2) == q) {
        const int i = tok & 3;
        h[(size_t)(p0 + p) * I + j] = i == 0 ? hv[0] : (i == 1 ? hv[1] : (i == 2 ? hv[2] : hv[3]));
      }
    }
  };
  compute_unit();
  // further units of the share (when it exceeds one per wave): the wave's
  // own scale slot is reused once its reads are done
  for (int uu = u0 + wv + WPB; uu < u1; uu += WPB) {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
    begin_unit(uu);
    wait_vmcnt<2 * D>();
    compute_unit();
  }
}

// The decode layer's first kernel: router top-K and permutation of the batch
// folded into the whole-CU gate_up (moe_layer).  Every block routes and
// permutes the T <= 8 tokens itself in LDS (a few microseconds of latency,
// the same in every block) instead of waiting for a separate launch; block 0
// also writes the permutation's outputs, which the down and combine kernels
// read after this kernel.  Meanwhile waves 8.. each stage one activation row
// by DMA and convert it, with no barrier (each converts what it loaded).
// Then the block takes its share of the active units as k_dec_gate_up_cu
// does, with the group metadata from LDS.  Same arithmetic as the separate
// launches, so the same bits (with KS > 1, the same bits as k_dec_gate_up's
// split of the same KS).  (Issuing each wave's first unit loads before the
// permutation's second half, from the union of the token bitmaps, measured
// slower: the waves then stall issuing into the full memory pipeline and the
// permutation ends about 3 us later at T = 8.)
// KS > 1 (split K, for launches whose blocks hold at most kGuCuWaves / KS
// units): the block's waves work in rounds of kGuCuWaves / KS units, KS
// consecutive waves per unit, each on NCH / KS consecutive chunks (all of
// them in flight at once) with the unit's scale runs in its own LDS slot;
// waves 1 .. KS-1 of a unit leave their partial sums in their slots, and
// after a barrier the unit's first wave adds them in wave order (a fixed
// order: the result does not depend on timing) and runs the epilogue.  Every wave takes part in every round's barriers.
template <int NCH, int TR, bool FP8, int MAXV, int KS>
__global__ __launch_bounds__(64 * kGuCuWaves) void k_dec_layer_gate_up(
    const float* __restrict__ logits, int E, const uint8_t* __restrict__ gu_codes,
    const uint8_t* __restrict__ gu_scales, const float* __restrict__ scale2,
    const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, float* __restrict__ xs, int T,
    int K, int H, int I, int has_shared, RpOut ro, uint16_t* __restrict__ h) {
  constexpr int WPB = kGuCuWaves;
  static_assert(WPB >= 8 + TR, "a converting wave per activation row");
  static_assert(NCH % KS == 0 && WPB % KS == 0, "whole chunks per wave, whole units per round");
  __shared__ RpLds L;
  extern __shared__ __align__(16) _Float16 xl[];
  constexpr int CPR = 16 * NCH;                     // 16-byte chunks per row, H = 128 * NCH
  constexpr int SRUN = 128 * NCH;                   // scale bytes of 16 rows
  constexpr int NCK = NCH / KS;                     // chunks per wave
  constexpr int D = KS > 1 ? NCK : (NCH < kGuPipe ? NCH : kGuPipe);  // chunks in flight
  constexpr int SLOT = dec_layer_slot_bytes(NCH, KS);
  const int lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ks = wv % KS, c0 = ks * NCK;            // this wave's part of K
  const bool blk0 = blockIdx.x == 0;
  float* fac = (float*)((uint8_t*)xl + (size_t)TR * H * 2);
  uint8_t* const slot0 = (uint8_t*)xl + (size_t)TR * H * 2 + 256;
  uint8_t* sl = slot0 + (size_t)wv * SLOT;

  // (1) waves 8 .. 8 + TR - 1: activation row wv - 8 -> LDS (chunk-swizzled),
  // then converted in place by the same wave
  if (wv >= 8 && wv - 8 < TR) {
    const int r = wv - 8;
    const uint16_t* xr_g = x + (size_t)(r < T ? r : T - 1) * H;
    for (int base = 0; base < CPR; base += 64) {
      const int ch = base + lane;
      if (ch < CPR)
        dma16(xr_g + 8 * (ch ^ (r & 15)), (uint8_t*)xl + 16 * ((size_t)r * CPR + base));
    }
    wait_vmcnt<0>();
    dec_convert_rows<CPR, TR, 8>(xl, fac, xs, xq, H, T, FP8, FP8 && blk0, r, lane);
  }
  // (2) waves < T route; (3) the block permutes (barriers inside, which also
  // publish the converted rows)
  rp_route<MAXV, 64 * WPB>(logits, T, E, K, has_shared, blk0, ro, L);
  const int nact = rp_permute<64 * WPB>(T, E, K, has_shared, blk0, ro, L);

  // (4) this block's share of the active units
  const int nbk = I / 16;
  const int units = nact * nbk;
  const int u0 = (int)((long long)blockIdx.x * units / gridDim.x);
  const int u1 = (int)((long long)(blockIdx.x + 1) * units / gridDim.x);
  const size_t rowb = (size_t)H / 2;
  int e = 0, pb = 0, p0 = 0, n = 1, slot_l = 0;
  float s2g = 0.f, s2u = 0.f;
  const uint8_t* cg = gu_codes;
  const uint8_t* cu = gu_codes;
  u32x4 wg[NCK], wu[NCK];
  auto issue = [&](int c) {
    wg[c] = *(const u32x4*)(cg + 64 * c);
    wu[c] = *(const u32x4*)(cu + 64 * c);
  };
  auto begin_unit = [&](int uu) {
    const int a = uu / nbk;
    pb = uu % nbk;
    e = __builtin_amdgcn_readfirstlane(L.gl[a]);
    const size_t grow = (size_t)e * 2 * I + (size_t)pb * 16;  // first gate row of the unit
    const uint8_t* sg = gu_scales + grow * (H / 16);
    dma_run<SRUN>(sg, sl, lane);
    dma_run<SRUN>(sg + (size_t)I * (H / 16), sl + SRUN, lane);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    p0 = __builtin_amdgcn_readfirstlane(L.run[e] & 0xFFFF);
    n = __builtin_amdgcn_readfirstlane(L.cnt[e]);
    s2g = scale2[3 * e + 0];
    s2u = scale2[3 * e + 1];
    slot_l = L.ss_l[p0 + (lane < n ? lane : n - 1)];
    cg = gu_codes + (grow + r16) * rowb + 16 * q + 64 * c0;
    cu = cg + (size_t)I * rowb;
#pragma unroll
    for (int c = 0; c < D; ++c) issue(c);
    __builtin_amdgcn_sched_barrier(0);
  };
  float ums[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) ums[t] = fac[t < TR ? t : TR - 1];
  const int xr = r16 < T ? r16 : T - 1;
  const uint8_t* xrow = (const uint8_t*)xl;
  const uint8_t* srow = sl + r16 * (8 * NCH) + 2 * q + 8 * c0;
  // the swizzle touches only the low 4 bits of the chunk index, so the
  // operand of sub-MFMA (c, j) sits at aoff[j] + 256 c
  int aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aoff[j] = swz_off(xr, 4 * q + j, CPR) + 256 * c0;
  // the MFMAs of this wave's chunks (chunk c once it has landed, then chunk
  // c + D is issued); the scale runs must have landed
  auto mma_unit = [&](f32x4& dg, f32x4& du) {
    static_for<0, NCK>([&](auto ct) {
      constexpr int c = decltype(ct)::value;
      constexpr int issued = D + c < NCK ? D + c : NCK;
      wait_vmcnt<2 * (issued - c - 1)>();
      const f16x2 sgv = e4m3x2_to_f16(*(const uint16_t*)(srow + 8 * c));
      const f16x2 suv = e4m3x2_to_f16(*(const uint16_t*)(srow + SRUN + 8 * c));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x8 av = *(const f16x8*)(xrow + aoff[j] + 256 * c);
        dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(wg[c][j], j < 2 ? sgv.x : sgv.y), dg, 0, 0, 0);
        du = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(wu[c][j], j < 2 ? suv.x : suv.y), du, 0, 0, 0);
      }
      if constexpr (c + D < NCK) issue(c + D);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto epilogue = [&](const f32x4& dg, const f32x4& du) {
    uint16_t hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float um = q == 0 ? ums[i] : (q == 1 ? ums[4 + i] : 0.f);  // tokens >= 8 are never stored
      const float g = dg[i] * um * s2g, u = du[i] * um * s2u;
      hv[i] = f32_to_bf16_bits(silu_f32(g) * u);
    }
    const int tokl = slot_token(slot_l, T, K, has_shared);
    const int j = pb * 16 + r16;
    for (int p = 0; p < n; ++p) {
      const int tok = p < 64 ? __shfl(tokl, p, 64) : slot_token(L.ss_l[p0 + p], T, K, has_shared);
      if (tok >= 0 && (tok >> 2) == q) {
        const int i = tok & 3;
        h[(size_t)(p0 + p) * I + j] = i == 0 ? hv[0] : (i == 1 ? hv[1] : (i == 2 ? hv[2] : hv[3]));
      }
    }
  };
  if constexpr (KS == 1) {
    for (int uu = u0 + wv; uu < u1; uu += WPB) {  // uniform per wave; no barrier follows
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
      begin_unit(uu);
      wait_vmcnt<2 * D>();  // the scale runs have landed
      f32x4 dg = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
      mma_unit(dg, du);
      epilogue(dg, du);
    }
  } else {
    constexpr int UPR = WPB / KS;                  // units per round
    const int rounds = (u1 - u0 + UPR - 1) / UPR;  // uniform per block
    for (int rd = 0; rd < rounds; ++rd) {
      const int uu = u0 + rd * UPR + wv / KS;
      const bool has = uu < u1;                    // uniform per wave
      if (rd > 0) __syncthreads();                 // the last round's partial sums are read
      f32x4 dg = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
      if (has) {
        begin_unit(uu);
        wait_vmcnt<2 * D>();
        mma_unit(dg, du);
        if (ks > 0) {  // partial sums -> this wave's slot ([8][64] floats, lane fastest)
          float* dst = (float*)sl + lane;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dst[64 * i] = dg[i];
            dst[64 * (4 + i)] = du[i];
          }
        }
      }
      __syncthreads();
      if (has && ks == 0) {
#pragma unroll
        for (int w = 1; w < KS; ++w) {
          const float* src = (const float*)(sl + (size_t)w * SLOT) + lane;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dg[i] += src[64 * i];
            du[i] += src[64 * (4 + i)];
          }
        }
        epilogue(dg, du);
      }
    }
  }
}

// --------------------------------- down -----------------------------------
// One wave = one unit (group, 16 NB output rows as NB MFMA blocks of 16, all
// of K = I); a block holds WPB consecutive units of one group and the group's
// h rows (up to 16 per pass) in LDS, chunk-swizzled like the activations
// above.  Code loads are row-contiguous as in gate_up (lane (r16, q), chunk
// c: bytes 64c + 16q of the row); the unit's block scales are one contiguous
// run that goes to LDS by DMA.  Every position of a group's range is a valid
// slot (the permutation only places valid ones), so the rows are read without
// a slot lookup.  Only the pass's valid rows are staged: the MFMA rows past
// them read whatever the LDS holds, and their outputs (each output row
// depends on its own A row only) are not stored.
// Dynamic LDS: [16][I] h rows (bf16 as loaded, f16 after the conversion),
// then per wave the scale run (16 NB x I/16 B), then the 16 rows' epilogue
// factors (f32).
template <int NCH, int WPB, int NB>   // NCH = I / 128
__global__ __launch_bounds__(64 * WPB) void k_dec_down(
    const uint8_t* __restrict__ dn_codes, const uint8_t* __restrict__ dn_scales,
    const float* __restrict__ scale2, const uint16_t* __restrict__ h,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ groups, int H, int I,
    uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) uint16_t hl[];
  constexpr int SRUN = 128 * NB * NCH;  // scale bytes of the unit's 16 NB rows
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, r16 = lane & 15, q = lane >> 4;
  const int cpr = I / 8;
  const int nbk = H / (16 * NB) / WPB;
  const int a = blockIdx.x / nbk, rb = (blockIdx.x % nbk) * WPB + wv;
  const int nact = groups[0], e = groups[1 + a];
  asm volatile("" ::"s"(e));  // both lookups in one trip
  if (a >= nact) return;      // uniform per block
  const int p0 = offsets[e], n = offsets[e + 1] - p0;  // scalar loads, in flight meanwhile
  uint8_t* sl = (uint8_t*)hl + (size_t)16 * I * 2 + (size_t)wv * SRUN;
  const size_t row0 = (size_t)e * H + (size_t)rb * 16 * NB;
  const size_t rowb = (size_t)I / 2;
  const uint8_t* cr = dn_codes + (row0 + r16) * rowb + 16 * q;
  u32x4 w[NB][NCH];
  // chunks [c0, c1) of every row block, issued in the order the MFMAs use them
  auto load_codes = [&](auto c0t, auto c1t) {
    constexpr int c0 = decltype(c0t)::value, c1 = decltype(c1t)::value;
#pragma unroll
    for (int c = c0; c < c1; ++c) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) w[nb][c] = *(const u32x4*)(cr + (size_t)nb * 16 * rowb + 64 * c);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the group's valid h rows of [r0, r0 + 16) -> LDS
  auto stage = [&](int r0) {
    const int nv = n - r0 < 16 ? n - r0 : 16;
    dma_rows_swizzled(hl, nv, cpr, wv, WPB, lane,
                      [&](int r) { return (const uint8_t*)(h + (size_t)(p0 + r0 + r) * I); });
  };
  // Issue order: scale run, h rows of the first pass, the first DD code
  // chunks; the rest are issued one by one as the first pass consumes chunks
  // (software pipelining, as in gate_up: the h rows land before the weight
  // stream fills the memory pipeline, and the MFMAs run while it streams).
  constexpr int DD = NCH < kDnPipe ? NCH : kDnPipe;
  dma_run<SRUN>(dn_scales + row0 * (I / 16), sl, lane);
  stage(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);  // the code loads stay behind the h rows
  load_codes(std::integral_constant<int, 0>(), std::integral_constant<int, DD>());
  const float s2d = scale2[3 * e + 2];
  const uint8_t* hrow = (const uint8_t*)hl;
  const uint8_t* srow = sl + r16 * (8 * NCH) + 2 * q;
  // A operand of sub-MFMA (c, j) at haoff[j] + 256 c (the swizzle touches only
  // the low 4 bits of the chunk index)
  int haoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) haoff[j] = swz_off(r16, 4 * q + j, cpr);
  float* hfac = (float*)((uint8_t*)hl + (size_t)16 * I * 2 + (size_t)WPB * SRUN);  // [16]
  // The staged bf16 h rows of a pass -> f16 in place, each row times the
  // power of two that brings its absmax into [2^14, 2^15) (the rule of the
  // activation rows in gate_up), undone in the epilogue; rows past the
  // group's end are left as they are (their outputs are never stored).
  constexpr int NCLD = (16 * NCH + 63) / 64;  // 16-byte chunks of a row per lane
  auto convert_h = [&](int r0) {
    const int nv = n - r0 < 16 ? n - r0 : 16;  // valid rows of the pass
    for (int r = wv; r < nv; r += WPB) {
      u32x4 v[NCLD];
#pragma unroll
      for (int k = 0; k < NCLD; ++k) {
        const int ch = lane + 64 * k;
        v[k] = ch < cpr ? *(const u32x4*)(hrow + swz_off(r, ch, cpr)) : u32x4{0u, 0u, 0u, 0u};
      }
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < NCLD; ++k)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[k][jj] & 0xFFFFu)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[k][jj] >> 16)));
        }
      amax = wave_max_nonneg(amax);  // fmaxf drops NaN: every lane is >= 0, not NaN
      const int sh = f16_row_shift(amax);
      const float mul = ldexpf(1.0f, sh);
      if (lane == 0) hfac[r] = ldexpf(1.0f, -sh);
#pragma unroll
      for (int k = 0; k < NCLD; ++k) {
        const int ch = lane + 64 * k;
        if (ch >= cpr) break;
        u32x4 o;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          o[jj] = pack_f16x2(bf16_bits_to_f32(v[k][jj] & 0xFFFFu) * mul,
                             bf16_bits_to_f32(v[k][jj] >> 16) * mul);
        *(u32x4*)((uint8_t*)hl + swz_off(r, ch, cpr)) = o;
      }
    }
  };
  auto mfma_chunk = [&](f32x4 (&acc)[NB], int c) {
    f16x2 sc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      sc[nb] = e4m3x2_to_f16(*(const uint16_t*)(srow + nb * 16 * (8 * NCH) + 8 * c));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x8 av = __builtin_bit_cast(f16x8, *(const u32x4*)(hrow + haoff[j] + 256 * c));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(w[nb][c][j], j < 2 ? sc[nb].x : sc[nb].y), acc[nb], 0, 0, 0);
    }
  };
  auto epilogue = [&](const f32x4 (&acc)[NB], int r0) {
    float rf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rf[i] = hfac[4 * q + i];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = rb * 16 * NB + nb * 16 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mm = 4 * q + i;
        if (r0 + mm < n) y[(size_t)(p0 + r0 + mm) * H + col] = f32_to_bf16_bits(acc[nb][i] * rf[i] * s2d);
      }
    }
  };
  // every code chunk loaded: one pass over all of them
  auto compute = [&](int r0) {
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      mfma_chunk(acc, c);
      // keep each chunk's dequantised operands next to their MFMAs (bounds
      // the registers in flight)
      __builtin_amdgcn_sched_barrier(0);
    }
    epilogue(acc, r0);
  };
  // this wave's DMAs are complete once only the first code chunks are
  // outstanding; the barrier covers the block
  wait_vmcnt<NB * DD>();
  __builtin_amdgcn_s_barrier();
  convert_h(0);
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  {  // first pass: chunk c once it has landed, then issue chunk c + DD
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    static_for<0, NCH>([&](auto ct) {
      constexpr int c = decltype(ct)::value;
      constexpr int issued = DD + c < NCH ? DD + c : NCH;
      wait_vmcnt<NB * (issued - c - 1)>();
      mfma_chunk(acc, c);
      if constexpr (c + DD < NCH)
        load_codes(std::integral_constant<int, c + DD>(), std::integral_constant<int, c + DD + 1>());
      __builtin_amdgcn_sched_barrier(0);
    });
    epilogue(acc, 0);
  }
  for (int r0 = 16; r0 < n; r0 += 16) {  // only when ids repeat (> 16 rows)
    __syncthreads();  // previous pass done reading hl and hfac
    stage(r0);
    __syncthreads();
    convert_h(r0);
    __syncthreads();
    // the code words count as redefined on every pass, so the dequantised
    // operands (4x the registers of the codes) are not hoisted out of the loop
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < NCH; ++c) asm volatile("" : "+v"(w[nb][c]));
    compute(r0);
  }
}

// ------------------------- down + combine (small T) ------------------------
// The decode layer's down and combine in one launch, for batches routed by
// the layer itself: the K experts of a token are distinct, so a group holds
// at most T positions (TR = T rounded up to 1, 2, 4 or 8 rows).  Block b takes
// the output columns [16 b, 16 b + 16) of every active group; wave w takes
// groups w, w + kDcWaves, ... and computes each exactly as a 16-row
// k_dec_down unit does (the group's h rows staged and converted with the same
// per-row power of two, in this wave's own LDS region; the same MFMA order
// and epilogue), so y has the same bits; it writes y and keeps a copy of its
// rows in LDS.  After one barrier the block combines its 16 columns of every
// token from that copy (combine_rows: the combine kernel's arithmetic, the
// same bits).  No block waits for another.
// Dynamic LDS: per wave [TR][I] h rows; per wave 16 row factors (f32); per
// wave the unit's scale run (16 x I/16 B); then the y copy [S][16] (bf16).
constexpr int kDcWaves = 16;

template <int NCH, int TR>   // NCH = I / 128
__global__ __launch_bounds__(64 * kDcWaves) void k_dec_down_combine(
    const uint8_t* __restrict__ dn_codes, const uint8_t* __restrict__ dn_scales,
    const float* __restrict__ scale2, const uint16_t* __restrict__ h,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ groups,
    const float* __restrict__ w, const int32_t* __restrict__ slot_pos,
    const float* __restrict__ gate, int T, int K, int H, int I, int has_shared,
    uint16_t* __restrict__ y, uint16_t* __restrict__ out) {
  constexpr int WPB = kDcWaves;
  constexpr int CPR = 16 * NCH;       // 16-byte chunks of an h row
  constexpr int SRUN = 128 * NCH;     // scale bytes of 16 rows
  constexpr int HW = TR * CPR * 16;   // bytes of a wave's h rows
  constexpr int NCLD = (CPR + 63) / 64;
  extern __shared__ __align__(16) uint8_t dl[];
  const int lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* hw = dl + (size_t)wv * HW;
  float* hfac = (float*)(dl + (size_t)WPB * HW) + 16 * wv;
  uint8_t* sl = dl + (size_t)WPB * HW + WPB * 64 + (size_t)wv * SRUN;
  uint16_t* yl = (uint16_t*)(dl + (size_t)WPB * (HW + 64 + SRUN));
  const int col0 = blockIdx.x * 16;
  const int nact = groups[0];
  const size_t rowb = (size_t)I / 2;
  // A operand of sub-MFMA (c, j) at haoff[j] + 256 c; MFMA rows past TR read
  // row TR - 1 (their outputs are never stored)
  const int xr = r16 < TR ? r16 : TR - 1;
  int haoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) haoff[j] = swz_off(xr, 4 * q + j, CPR);
  const uint8_t* srow = sl + r16 * (8 * NCH) + 2 * q;
  for (int a = wv; a < nact; a += WPB) {  // uniform per wave
    const int e = __builtin_amdgcn_readfirstlane(groups[1 + a]);
    const int p0 = __builtin_amdgcn_readfirstlane(offsets[e]);
    // n <= T <= TR by the routing; the clamp only keeps LDS in bounds
    const int nn = __builtin_amdgcn_readfirstlane(offsets[e + 1]) - p0;
    const int n = nn < TR ? nn : TR;
    const size_t row0 = (size_t)e * H + col0;
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): the last group's LDS reads
    // scale run, the group's h rows, then every code chunk
    dma_run<SRUN>(dn_scales + row0 * (I / 16), sl, lane);
    dma_rows_swizzled(hw, n, CPR, 0, 1, lane,
                      [&](int r) { return (const uint8_t*)(h + (size_t)(p0 + r) * I); });
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    u32x4 wc[NCH];
    const uint8_t* cr = dn_codes + (row0 + r16) * rowb + 16 * q;
#pragma unroll
    for (int c = 0; c < NCH; ++c) wc[c] = *(const u32x4*)(cr + 64 * c);
    __builtin_amdgcn_sched_barrier(0);
    const float s2d = scale2[3 * e + 2];
    wait_vmcnt<NCH>();  // the scale run and the h rows have landed
    // the h rows -> f16 in place, each times the power of two that brings its
    // absmax into [2^14, 2^15), undone in the epilogue (k_dec_down's rule)
    for (int r = 0; r < n; ++r) {
      u32x4 v[NCLD];
#pragma unroll
      for (int k = 0; k < NCLD; ++k) {
        const int ch = lane + 64 * k;
        v[k] = ch < CPR ? *(const u32x4*)(hw + swz_off(r, ch, CPR)) : u32x4{0u, 0u, 0u, 0u};
      }
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < NCLD; ++k)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[k][jj] & 0xFFFFu)));
          amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[k][jj] >> 16)));
        }
      amax = wave_max_nonneg(amax);  // fmaxf drops NaN: every lane is >= 0, not NaN
      const int sh = f16_row_shift(amax);
      const float mul = ldexpf(1.0f, sh);
      if (lane == 0) hfac[r] = ldexpf(1.0f, -sh);
#pragma unroll
      for (int k = 0; k < NCLD; ++k) {
        const int ch = lane + 64 * k;
        if (ch >= CPR) break;
        u32x4 o;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          o[jj] = pack_f16x2(bf16_bits_to_f32(v[k][jj] & 0xFFFFu) * mul,
                             bf16_bits_to_f32(v[k][jj] >> 16) * mul);
        *(u32x4*)(hw + swz_off(r, ch, CPR)) = o;
      }
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    static_for<0, NCH>([&](auto ct) {
      constexpr int c = decltype(ct)::value;
      wait_vmcnt<NCH - c - 1>();
      const f16x2 sc = e4m3x2_to_f16(*(const uint16_t*)(srow + 8 * c));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x8 av = __builtin_bit_cast(f16x8, *(const u32x4*)(hw + haoff[j] + 256 * c));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(wc[c][j], j < 2 ? sc.x : sc.y), acc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mm = 4 * q + i;
      if (mm < n) {
        const uint16_t v = f32_to_bf16_bits(acc[i] * hfac[mm] * s2d);
        y[(size_t)(p0 + mm) * H + col0 + r16] = v;
        yl[(size_t)(p0 + mm) * 16 + r16] = v;
      }
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < 2 * T) {  // token t, columns col0 + 8 half .. + 8
    const int t = threadIdx.x >> 1, half = threadIdx.x & 1;
    combine_rows([&](int pp) { return yl + (size_t)pp * 16 + 8 * half; }, w, slot_pos, gate, T, K,
                 has_shared, out + (size_t)t * H + col0 + 8 * half, t);
  }
}

// --------------------------------- host -----------------------------------

// The decode layer kernel's variants of one (NCH, TR, MAXV): K split over 1,
// 2, 4 or 8 waves (where NCH allows).
template <int NCH, int TR, int MV, int KS>
static void reg_dec_layer_gate_up1(std::vector<const void*>& k) {
  if constexpr (NCH % KS == 0) {
    k.push_back((const void*)&k_dec_layer_gate_up<NCH, TR, false, MV, KS>);
    k.push_back((const void*)&k_dec_layer_gate_up<NCH, TR, true, MV, KS>);
  }
}
template <int NCH, int TR, int MV>
static void reg_dec_layer_gate_up(std::vector<const void*>& k) {
  reg_dec_layer_gate_up1<NCH, TR, MV, 1>(k);
  reg_dec_layer_gate_up1<NCH, TR, MV, 2>(k);
  reg_dec_layer_gate_up1<NCH, TR, MV, 4>(k);
  reg_dec_layer_gate_up1<NCH, TR, MV, 8>(k);
}

void register_decode_kernels(std::vector<const void*>& k) {
  k.push_back((const void*)&k_dec_xprep<false>);
  k.push_back((const void*)&k_dec_xprep<true>);
#define MOE_REG_GU3(NCH, WPB, TR, KS)                                    \
  k.push_back((const void*)&k_dec_gate_up<NCH, WPB, TR, false, KS>); \
  k.push_back((const void*)&k_dec_gate_up<NCH, WPB, TR, true, KS>);
#define MOE_REG_GU2(NCH, WPB, KS) \
  MOE_REG_GU3(NCH, WPB, 1, KS)    \
  MOE_REG_GU3(NCH, WPB, 2, KS)    \
  MOE_REG_GU3(NCH, WPB, 4, KS)    \
  MOE_REG_GU3(NCH, WPB, 8, KS)
#define MOE_REG_GU(NCH)  \
  MOE_REG_GU2(NCH, 1, 1) \
  MOE_REG_GU2(NCH, 4, 1)
  MOE_REG_GU(2)
  MOE_REG_GU(4)
  MOE_REG_GU(8)
  MOE_REG_GU(16)
  MOE_REG_GU2(4, 4, 4)
  MOE_REG_GU2(8, 4, 4)
  MOE_REG_GU2(16, 4, 4)
#define MOE_REG_GUC2(NCH, TR)                                    \
  k.push_back((const void*)&k_dec_gate_up_cu<NCH, TR, false>); \
  k.push_back((const void*)&k_dec_gate_up_cu<NCH, TR, true>);
#define MOE_REG_GUC(NCH) \
  MOE_REG_GUC2(NCH, 1)   \
  MOE_REG_GUC2(NCH, 2)   \
  MOE_REG_GUC2(NCH, 4)   \
  MOE_REG_GUC2(NCH, 8)
  MOE_REG_GUC(2)
  MOE_REG_GUC(4)
  MOE_REG_GUC(8)
  MOE_REG_GUC(16)
#undef MOE_REG_GUC
#undef MOE_REG_GUC2
#define MOE_REG_LGU2(NCH, TR)                \
  reg_dec_layer_gate_up<NCH, TR, 8>(k); \
  reg_dec_layer_gate_up<NCH, TR, 16>(k);
#define MOE_REG_LGU(NCH) \
  MOE_REG_LGU2(NCH, 1)   \
  MOE_REG_LGU2(NCH, 2)   \
  MOE_REG_LGU2(NCH, 4)   \
  MOE_REG_LGU2(NCH, 8)
  MOE_REG_LGU(2)
  MOE_REG_LGU(4)
  MOE_REG_LGU(8)
  MOE_REG_LGU(16)
#undef MOE_REG_LGU
#undef MOE_REG_LGU2
#undef MOE_REG_GU
#undef MOE_REG_GU2
#undef MOE_REG_GU3
#define MOE_REG_DN(NCH)                              \
  k.push_back((const void*)&k_dec_down<NCH, 4, 4>); \
  k.push_back((const void*)&k_dec_down<NCH, 4, 2>); \
  k.push_back((const void*)&k_dec_down<NCH, 4, 1>);
  k.push_back((const void*)&k_dec_down<1, 4, 4>);
  k.push_back((const void*)&k_dec_down<1, 4, 2>);
  MOE_REG_DN(2)
  MOE_REG_DN(4)
  MOE_REG_DN(8)
#undef MOE_REG_DN
#define MOE_REG_DC(NCH)                                        \
  k.push_back((const void*)&k_dec_down_combine<NCH, 1>); \
  k.push_back((const void*)&k_dec_down_combine<NCH, 2>); \
  k.push_back((const void*)&k_dec_down_combine<NCH, 4>); \
  k.push_back((const void*)&k_dec_down_combine<NCH, 8>);
  MOE_REG_DC(2)
  MOE_REG_DC(4)
  MOE_REG_DC(8)
#undef MOE_REG_DC
}

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Shapes the decode kernels are instantiated for (others take the grouped path).
bool decode_supported(int H, int I) {
  const int nch = H / 128, ncd = I / 128;
  return (nch == 2 || nch == 4 || nch == 8 || nch == 16) &&
         (ncd == 1 || ncd == 2 || ncd == 4 || ncd == 8);
}

// One block per token row (H <= 4096): f16 rows and epilogue factors, and
// for the FP8 arm the e4m3 codes and row scales.
hipError_t launch_xprep(const uint16_t* x, int T, int H, bool fp8, _Float16* xh, float* unmul,
                        uint8_t* xq, float* xs, hipStream_t s) {
  if (fp8)
    MOE_LAUNCH("xprep", s, (k_dec_xprep<true>), dim3(T), dim3(256), 0, s, x, H, xh, unmul, xq, xs);
  else
    MOE_LAUNCH("xprep", s, (k_dec_xprep<false>), dim3(T), dim3(256), 0, s, x, H, xh, unmul, xq, xs);
  return hipGetLastError();
}

// f16 activation rows [T][H] and their epilogue factors [T] (grouped path).
size_t xprep_workspace_bytes(int T, int H) {
  return align256((size_t)T * H * sizeof(_Float16)) + align256((size_t)T * sizeof(float));
}

// gate_up launch for one (NCH, WPB, KS): picks the staged row count and the arm.
template <int NCH, int WPB, int KS>
static void launch_dec_gate_up(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                               const int32_t* offsets, const int32_t* sorted_slot,
                               const int32_t* groups, int act_mode, uint8_t* xq, float* xs,
                               uint16_t* hbuf, dim3 grid, hipStream_t s) {
  const bool fp8 = act_mode != MOE_ACT_BF16;
  const int fp8_sel = act_mode == MOE_ACT_FP8_ROUTED ? 1 : (act_mode == MOE_ACT_FP8_SHARED ? 2 : 0);
  const int shared_g = W.has_shared ? W.E : -1;
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const int tr = T <= 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8));  // activation rows staged
  const size_t lds = (size_t)tr * H * 2 + 256 +
                     (KS > 1 ? (size_t)2 * 16 * (H / 16) + (size_t)(KS - 1) * 512 * sizeof(float)
                             : (size_t)WPB * 2 * 16 * (H / 16));
#define MOE_DEC_GU1(TR, F8)                                                                           \
  MOE_LAUNCH("dec_gate_up", s, (k_dec_gate_up<NCH, WPB, TR, F8, KS>), grid, dim3(64 * WPB), lds, s,  \
             W.gu_codes, W.gu_scales, W.scale2, x, xq, xs, offsets, sorted_slot, groups, T, K, H, \
             I, hs, fp8_sel, shared_g, hbuf)
#define MOE_DEC_GU2(TR)                \
  do {                                 \
    if (fp8) MOE_DEC_GU1(TR, true);    \
    else MOE_DEC_GU1(TR, false);       \
  } while (0)
  if (tr == 1) MOE_DEC_GU2(1);
  else if (tr == 2) MOE_DEC_GU2(2);
  else if (tr == 4) MOE_DEC_GU2(4);
  else MOE_DEC_GU2(8);
#undef MOE_DEC_GU2
#undef MOE_DEC_GU1
}

// Split K below this many gate_up units per CU (see k_dec_gate_up).
constexpr long kGuSplitBelow = 2;
// K split of the decode layer kernel: at most kLayerSplitMaxKs waves per
// unit, and only while a block holds at most kLayerSplitMaxShare units.
// Measured at H = 2048, I = 512, E = 512, K = 10 (whole layer, weights cold):
// T = 1 23.8 -> 22.3 us (8 waves), T = 2 26.6 -> 25.8, T = 3 29.5 -> 29.1
// (4 waves); T = 4 33.4 / 33.5 and T = 6 41.4 / 42.1 with 2 waves.
constexpr long kLayerSplitMaxKs = 8;
constexpr long kLayerSplitMaxShare = 4;
// Whole-CU gate_up blocks (k_dec_gate_up_cu) from this many units per CU on.
constexpr long kGuCuFrom = 4;

// The whole-CU gate_up launch: one block per CU.
template <int NCH>
static void launch_gu_cu(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                         const int32_t* offsets, const int32_t* sorted_slot,
                         const int32_t* groups, int act_mode, uint8_t* xq, float* xs,
                         uint16_t* hbuf, hipStream_t s) {
  const bool fp8 = act_mode != MOE_ACT_BF16;
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const int tr = T <= 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8));
  const size_t lds = (size_t)tr * H * 2 + 256 + (size_t)kGuCuWaves * 2 * 16 * (H / 16);
  const dim3 grid((unsigned)num_cus()), block(64 * kGuCuWaves);
#define MOE_DEC_GUC1(TR, F8)                                                                     \
  MOE_LAUNCH("dec_gate_up", s, (k_dec_gate_up_cu<NCH, TR, F8>), grid, block, lds, s, W.gu_codes, \
             W.gu_scales, W.scale2, x, xq, xs, offsets, sorted_slot, groups, T, K, H, I, hs, hbuf)
#define MOE_DEC_GUC2(TR)              \
  do {                                \
    if (fp8) MOE_DEC_GUC1(TR, true);  \
    else MOE_DEC_GUC1(TR, false);     \
  } while (0)
  if (tr == 1) MOE_DEC_GUC2(1);
  else if (tr == 2) MOE_DEC_GUC2(2);
  else if (tr == 4) MOE_DEC_GUC2(4);
  else MOE_DEC_GUC2(8);
#undef MOE_DEC_GUC2
#undef MOE_DEC_GUC1
}
// Down units of 64 rows from this many per CU on, else of 32 or 16 rows
// (measured at H=2048, I=512, down us with the threshold at 0 / 4 / 8 / 16:
// T=1 7.1 / 6.9 / 6.5 / 6.3, T=4 10.4 / 10.1 / 9.6 / 9.2, T=8 13.7 / 13.4 /
// 13.5 / 12.3).
constexpr long kDnWavesPerCu = 16;

template <int NCH>
static void launch_gu_pick(bool split, int wpb, bool cu_mode, const moe_nvfp4_weights& W,
                           const uint16_t* x, int T, int K, const int32_t* offsets,
                           const int32_t* sorted_slot, const int32_t* groups, int act_mode,
                           uint8_t* xq, float* xs, uint16_t* hbuf, long units, hipStream_t s) {
  if (cu_mode) {
    launch_gu_cu<NCH>(W, x, T, K, offsets, sorted_slot, groups, act_mode, xq, xs, hbuf, s);
    return;
  }
  if constexpr (NCH % 4 == 0) {
    if (split) {
      launch_dec_gate_up<NCH, 4, 4>(W, x, T, K, offsets, sorted_slot, groups, act_mode, xq, xs,
                                    hbuf, dim3((unsigned)units), s);
      return;
    }
  }
  if (wpb == 4)
    launch_dec_gate_up<NCH, 4, 1>(W, x, T, K, offsets, sorted_slot, groups, act_mode, xq, xs,
                                  hbuf, dim3((unsigned)(units / 4)), s);
  else
    launch_dec_gate_up<NCH, 1, 1>(W, x, T, K, offsets, sorted_slot, groups, act_mode, xq, xs,
                                  hbuf, dim3((unsigned)units), s);
}

// The down launch of a decode FFN whose active groups number at most gmax.
static hipError_t launch_dec_down_all(const moe_nvfp4_weights& W, int gmax, const int32_t* offsets,
                                      const int32_t* groups, uint16_t* hbuf, uint16_t* y,
                                      hipStream_t s) {
  const int H = W.H, I = W.I;
  const long dn_units = (long)gmax * (H / 64);
  const long cus = num_cus();
  // Down rows per wave: 64 (4 MFMA blocks) once that gives kDnWavesPerCu
  // waves per CU, else 32 or 16 (more, shorter units at small T).
  // (A block is 4 waves = 64 NB rows of one group either way.)
  int nb_d = dn_units >= kDnWavesPerCu * cus ? 4 : (2 * dn_units >= kDnWavesPerCu * cus ? 2 : 1);
  if (nb_d * I < 256) nb_d = 2;  // the unit's scale run is whole DMA instructions (I = 128)
  const dim3 g2((unsigned)(dn_units * 4 / nb_d / 4)), b2(256);
  const size_t lds_dn = (size_t)16 * I * sizeof(uint16_t) + (size_t)4 * nb_d * I + 16 * sizeof(float);
  const int ncd = I / 128;
#define MOE_DEC_DN2(NCH, WPB, NB)                                                                 \
  MOE_LAUNCH("dec_down", s, (k_dec_down<NCH, WPB, NB>), g2, b2, lds_dn, s, W.dn_codes, W.dn_scales, \
             W.scale2, hbuf, offsets, groups, H, I, y)
#define MOE_DEC_DN(NCH)                          \
  do {                                           \
    if (nb_d == 4) MOE_DEC_DN2(NCH, 4, 4);       \
    else if (nb_d == 2) MOE_DEC_DN2(NCH, 4, 2);  \
    else MOE_DEC_DN2(NCH, 4, 1);                 \
  } while (0)
  if (ncd == 1) {
    if (nb_d == 4) MOE_DEC_DN2(1, 4, 4);
    else MOE_DEC_DN2(1, 4, 2);
  } else if (ncd == 2) MOE_DEC_DN(2);
  else if (ncd == 4) MOE_DEC_DN(4);
  else if (ncd == 8) MOE_DEC_DN(8);
  else return hipErrorInvalidValue;
#undef MOE_DEC_DN2
#undef MOE_DEC_DN
  return hipGetLastError();
}

hipError_t launch_decode_ffn(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                             const int32_t* offsets, const int32_t* sorted_slot,
                             const int32_t* groups, int act_mode, uint16_t* hbuf, uint8_t* xq,
                             float* xs, uint16_t* y, hipStream_t s) {
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const int G = W.E + hs;
  const int gmax = (int)((long)T * K + hs < (long)G ? (long)T * K + hs : (long)G);
  // gate_up waves (units) per block: 4 (one staged copy of the activation
  // rows per 4 units) once the units are plentiful, else 1 so that small T
  // still spreads over many CUs (measured at H=2048, I=512, 256 CUs: 4 gains
  // from about 2 units per CU on, T=3: 15.8 vs 17.8 us, T=6: 22.3 vs 37 us);
  // fewer than kGuSplitBelow units per CU: one unit per block with K split
  // over 4 waves (H a multiple of 512).
  const long gu_units = (long)gmax * (I / 16);
  const long cus = num_cus();
  const int wpb_g = gu_units >= 2 * cus ? 4 : 1;
  const bool split = gu_units < kGuSplitBelow * cus && (H / 128) % 4 == 0;
  // whole-CU blocks once every CU gets several units (one activation form
  // per block: the bf16 arm or the FP8 row arm)
  const bool cu_mode = !split && gu_units >= kGuCuFrom * cus &&
                       (act_mode == MOE_ACT_BF16 || act_mode == MOE_ACT_FP8_ROW);
  const int nch = H / 128;
#define MOE_DEC_GU(NCH)                                                                             \
  launch_gu_pick<NCH>(split, wpb_g, cu_mode, W, x, T, K, offsets, sorted_slot, groups, act_mode, \
                      xq, xs, hbuf, gu_units, s)
  if (nch == 2) MOE_DEC_GU(2);
  else if (nch == 4) MOE_DEC_GU(4);
  else if (nch == 8) MOE_DEC_GU(8);
  else if (nch == 16) MOE_DEC_GU(16);
  else return hipErrorInvalidValue;
#undef MOE_DEC_GU
  return launch_dec_down_all(W, gmax, offsets, groups, hbuf, y, s);
}

bool decode_layer_supported(int T, int E, int K, int H, int I, int act_mode) {
  return T >= 1 && T <= kRouteFuseMaxT && E <= kRpMaxE && K <= 32 && decode_supported(H, I) &&
         (act_mode == MOE_ACT_BF16 || act_mode == MOE_ACT_FP8_ROW);
}

// The decode layer kernel for one (NCH, TR, FP8, MAXV) and the K split `ks`.
template <int NCH, int TR, bool F8, int MV>
static void launch_dec_layer_gu(int ks, const moe_nvfp4_weights& W, const float* logits,
                                const uint16_t* x, int T, int K, const RpOut& ro, uint16_t* hbuf,
                                uint8_t* xq, float* xs, hipStream_t s) {
  const int H = W.H, I = W.I, E = W.E, hs = W.has_shared ? 1 : 0;
  const dim3 grid((unsigned)num_cus()), block(64 * kGuCuWaves);
  const size_t lds = (size_t)TR * H * 2 + 256 + (size_t)kGuCuWaves * dec_layer_slot_bytes(NCH, ks);
#define MOE_DEC_LGU0(KS)                                                                     \
  MOE_LAUNCH("dec_gate_up", s, (k_dec_layer_gate_up<NCH, TR, F8, MV, KS>), grid, block, lds, \
             s, logits, E, W.gu_codes, W.gu_scales, W.scale2, x, xq, xs, T, K, H, I, hs, ro, hbuf)
  if constexpr (NCH % 8 == 0) {
    if (ks == 8) { MOE_DEC_LGU0(8); return; }
  }
  if constexpr (NCH % 4 == 0) {
    if (ks == 4) { MOE_DEC_LGU0(4); return; }
  }
  if (ks == 2) MOE_DEC_LGU0(2);
  else MOE_DEC_LGU0(1);
#undef MOE_DEC_LGU0
}

// Down + combine of the decode layer in one launch (k_dec_down_combine) up
// to this many active groups; above it the down kernel's more, shorter units
// and the combine kernel.  Measured at H = 2048, I = 512, E = 512, K = 10
// (whole layer, weights cold), fused / separate: T = 1 16.7 / 18.7 us, T = 2
// 21.3 / 22.3, T = 4 29.6 / 29.7, T = 6 36.6 / 36.6, T = 8 44.3 / 41.9 (the
// fused launch has H / 16 blocks, too few once every group is long).
constexpr int kDcMaxGroups = 48;

// Dynamic LDS of k_dec_down_combine: per wave TR h rows, 16 row factors and
// a scale run; the y copy of the S slots' 16 columns.
static size_t dec_down_combine_lds(int T, int K, int I, int hs) {
  const int tr = T <= 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8));
  const size_t S = (size_t)T * K + (hs ? (size_t)T : 0);
  return (size_t)kDcWaves * ((size_t)tr * I * 2 + 64 + (size_t)I) + S * 32;
}
// Whether k_dec_down_combine takes this launch: I / 128 in {2, 4, 8}, H a
// multiple of 16, at most kDcMaxGroups groups, its LDS within the CU's.
static bool dec_down_combine_ok(int T, int K, int H, int I, int hs, int gmax) {
  const int ncd = I / 128;
  return (ncd == 2 || ncd == 4 || ncd == 8) && H % 16 == 0 && gmax <= kDcMaxGroups &&
         dec_down_combine_lds(T, K, I, hs) <= (size_t)160 * 1024;
}

static hipError_t launch_dec_down_combine(const moe_nvfp4_weights& W, int T, int K,
                                          const float* gate, const RpOut& ro,
                                          const uint16_t* hbuf, uint16_t* y, uint16_t* out,
                                          hipStream_t s) {
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const int tr = T <= 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8));
  const size_t lds = dec_down_combine_lds(T, K, I, hs);
  const dim3 grid((unsigned)(H / 16)), block(64 * kDcWaves);
  const int ncd = I / 128;
#define MOE_DEC_DC0(NCH, TR)                                                                       \
  MOE_LAUNCH("dec_down", s, (k_dec_down_combine<NCH, TR>), grid, block, lds, s, W.dn_codes,       \
             W.dn_scales, W.scale2, hbuf, ro.offsets, ro.groups, ro.w, ro.slot_pos, gate, T, K, H, \
             I, hs, y, out)
#define MOE_DEC_DC(NCH)                    \
  do {                                     \
    if (tr == 1) MOE_DEC_DC0(NCH, 1);      \
    else if (tr == 2) MOE_DEC_DC0(NCH, 2); \
    else if (tr == 4) MOE_DEC_DC0(NCH, 4); \
    else MOE_DEC_DC0(NCH, 8);              \
  } while (0)
  if (ncd == 2) MOE_DEC_DC(2);
  else if (ncd == 4) MOE_DEC_DC(4);
  else if (ncd == 8) MOE_DEC_DC(8);
  else return hipErrorInvalidValue;
#undef MOE_DEC_DC
#undef MOE_DEC_DC0
  return hipGetLastError();
}

// One block per CU: routing + permutation + gate_up (k_dec_layer_gate_up),
// then down and combine (k_dec_down_combine, or the down and combine
// kernels).  When a block's share of units is at most
// kLayerSplitMaxShare, the K split is the largest of 8, 4, 2 (dividing
// H / 128, at most kLayerSplitMaxKs) whose waves cover every unit of the
// share in one round; the share is bounded with the most groups the batch
// can activate, min(T K, E) (+ the shared expert).
hipError_t launch_decode_layer(const moe_nvfp4_weights& W, const float* logits, const uint16_t* x,
                               int T, int K, int act_mode, const float* gate, const RpOut& ro,
                               uint16_t* hbuf, uint8_t* xq, float* xs, uint16_t* y,
                               uint16_t* out, hipStream_t s) {
  const int H = W.H, I = W.I, E = W.E, hs = W.has_shared ? 1 : 0;
  const int G = E + hs;
  const int gmax = (int)((long)T * K + hs < (long)G ? (long)T * K + hs : (long)G);
  const bool fp8 = act_mode != MOE_ACT_BF16;
  const int tr = T <= 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8));
  const int nch = H / 128;
  const long units = (long)gmax * (I / 16);
  const long share = (units + num_cus() - 1) / num_cus();
  int ks = 1;
  if (share <= kLayerSplitMaxShare)
    while (2 * ks <= kLayerSplitMaxKs && 2 * ks * share <= kGuCuWaves && nch % (2 * ks) == 0) ks *= 2;
#define MOE_DEC_LGU2(NCH, TR)                                                                     \
  do {                                                                                            \
    if (E <= 512) {                                                                               \
      if (fp8) launch_dec_layer_gu<NCH, TR, true, 8>(ks, W, logits, x, T, K, ro, hbuf, xq, xs, s);   \
      else launch_dec_layer_gu<NCH, TR, false, 8>(ks, W, logits, x, T, K, ro, hbuf, xq, xs, s);      \
    } else {                                                                                      \
      if (fp8) launch_dec_layer_gu<NCH, TR, true, 16>(ks, W, logits, x, T, K, ro, hbuf, xq, xs, s);  \
      else launch_dec_layer_gu<NCH, TR, false, 16>(ks, W, logits, x, T, K, ro, hbuf, xq, xs, s);     \
    }                                                                                             \
  } while (0)
#define MOE_DEC_LGU(NCH)                    \
  do {                                      \
    if (tr == 1) MOE_DEC_LGU2(NCH, 1);      \
    else if (tr == 2) MOE_DEC_LGU2(NCH, 2); \
    else if (tr == 4) MOE_DEC_LGU2(NCH, 4); \
    else MOE_DEC_LGU2(NCH, 8);              \
  } while (0)
  if (nch == 2) MOE_DEC_LGU(2);
  else if (nch == 4) MOE_DEC_LGU(4);
  else if (nch == 8) MOE_DEC_LGU(8);
  else if (nch == 16) MOE_DEC_LGU(16);
  else return hipErrorInvalidValue;
#undef MOE_DEC_LGU
#undef MOE_DEC_LGU2
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (dec_down_combine_ok(T, K, H, I, hs, gmax))
    return launch_dec_down_combine(W, T, K, gate, ro, hbuf, y, out, s);
  err = launch_dec_down_all(W, gmax, ro.offsets, ro.groups, hbuf, y, s);
  if (err != hipSuccess) return err;
  return launch_combine(y, ro.w, ro.slot_pos, gate, T, K, H, hs, out, s);
}

}  // namespace moe
