// Decode/verify expert FFN (T <= 8 tokens): a multi-row GEMV on MFMA that
// streams each active expert's NVFP4 weights once (gate+up fused with SiLU,
// then down; routed experts and the shared expert in the same launches).
//
// The work is memory-bound, so the design maximises bytes in flight: one wave
// is one work unit and covers the whole K of its rows, issuing every weight
// load of the unit (code chunks and block scales) before its first MFMA.  No
// split-K, no cross-wave reduction, no loop-carried prefetch (the compiler
// drains all outstanding loads at such a loop's back edge).  Many resident
// waves per CU then keep HBM busy; a block holds 1 wave when the units would
// not fill the chip and 4 (one LDS copy of the activations) when they would.
//
// k_dec_xprep, once per layer call: each token row of x becomes f16 with a
// power-of-two shift (bf16 arm; the shift is undone in the f32 epilogue, see
// f16_row_shift) or, for the FP8 arm, is quantised to e4m3 per row and kept as
// the (exact) f16 value of each code, with the row scale as epilogue factor.
//
// k_dec_gate_up: unit = (active group, 16 gate/up row pairs).  The MFMA runs
// over the rows of ALL T tokens (T <= 8 of its 16 rows) and the epilogue keeps
// the tokens routed to the group, so the activation rows go to LDS before the
// group is even known.  f16 MFMA 16x16x32; weights are dequantised to f16
// exactly with one instruction per element.
//
// k_dec_down: unit = (active group, 64 output rows as 4 MFMA blocks of 16);
// A = the group's h rows (bf16, by sorted position), up to 16 per pass, in
// LDS; bf16 MFMA 16x16x32.
//
// Lane (r = l%16, q = l/16) of either kernel: B column r = weight row, A row r
// = token row (or group row); the lane owns the contiguous quarter
// [Q*q, Q*q + Q) of K (Q = K/4), read as 16-byte chunks of 32 elements, and
// 32-bit word j of chunk c feeds sub-MFMA (c, j): MFMA k index 8q + i maps to
// element Q*q + 32c + 8j + i on both operands, so the sum is over all of K.
#include "moe_ffn_common.hpp"
#include "moe_internal.hpp"

namespace moe {

// ------------------------------- x prep ------------------------------------

template <bool FP8>
__global__ __launch_bounds__(256) void k_dec_xprep(const uint16_t* __restrict__ x, int H,
                                                   _Float16* __restrict__ xh,
                                                   float* __restrict__ unmul,
                                                   uint8_t* __restrict__ xq,
                                                   float* __restrict__ xs) {
  __shared__ float wmax[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const u32x4* row = (const u32x4*)(x + (size_t)t * H);
  u32x4 v[2];
  float amax = 0.f;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int c = tid + 256 * cc;
    if (c < H / 8) {
      v[cc] = row[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[cc][j] & 0xFFFFu)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[cc][j] >> 16)));
      }
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float mul;
  if (FP8) {
    // the row quantisation of the FP8 arm (same rule as k_rowquant_e4m3)
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    mul = amax > 0.f ? 448.0f / amax : 1.0f;
    if (tid == 0) {
      xs[t] = s;
      unmul[t] = s;
    }
  } else {
    const int sh = f16_row_shift(amax);
    mul = ldexpf(1.0f, sh);
    if (tid == 0) unmul[t] = ldexpf(1.0f, -sh);
  }
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int c = tid + 256 * cc;
    if (c < H / 8) {
      u32x4 o;
      if (FP8) {
        u32x2 code;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float f0 = bf16_bits_to_f32(v[cc][2 * j] & 0xFFFFu) * mul;
          float f1 = bf16_bits_to_f32(v[cc][2 * j] >> 16) * mul;
          float f2 = bf16_bits_to_f32(v[cc][2 * j + 1] & 0xFFFFu) * mul;
          float f3 = bf16_bits_to_f32(v[cc][2 * j + 1] >> 16) * mul;
          f0 = fminf(fmaxf(f0, -448.f), 448.f);
          f1 = fminf(fmaxf(f1, -448.f), 448.f);
          f2 = fminf(fmaxf(f2, -448.f), 448.f);
          f3 = fminf(fmaxf(f3, -448.f), 448.f);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, w, true);
          code[j] = (uint32_t)w;
        }
        *(u32x2*)(xq + (size_t)t * H + 8 * c) = code;
        const u32x2 lo = fp8x4_to_f16(code.x), hi = fp8x4_to_f16(code.y);
        o = u32x4{lo.x, lo.y, hi.x, hi.y};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = pack_f16x2(bf16_bits_to_f32(v[cc][j] & 0xFFFFu) * mul,
                            bf16_bits_to_f32(v[cc][j] >> 16) * mul);
      }
      *(u32x4*)(xh + (size_t)t * H + 8 * c) = o;
    }
  }
}

// ------------------------------- gate_up ----------------------------------
// One wave = one unit (group, 16 gate/up row pairs, all of K); a block holds
// WPB waves = WPB consecutive units of one group and one LDS copy of the f16
// activation rows.  K is split between the 4 lane groups q of the wave in
// contiguous quarters: lane (r16, q) owns elements [Q*q, Q*q + Q) of weight row
// r16, Q = H/4, read as 16-byte code chunks (32 elements, one 128-element step
// per 4 chunks); its Q/16 block scales are contiguous bytes.

template <int NCH>   // NCH = 16-byte code chunks per lane per row = H / 128
struct GURegs {
  u32x4 g[NCH], u[NCH];
  // the lane's 2*NCH scale bytes: 16-byte loads when NCH is a multiple of 8,
  // else one 2-byte load per chunk (never past the lane's own bytes)
  static constexpr int NS = NCH % 8 == 0 ? NCH / 8 : NCH;
  u32x4 sg[NCH % 8 == 0 ? NCH / 8 : 1], su[NCH % 8 == 0 ? NCH / 8 : 1];
  uint32_t sg2[NCH % 8 == 0 ? 1 : NCH], su2[NCH % 8 == 0 ? 1 : NCH];
};

// scale bytes 2c, 2c+1 of the lane's contiguous run
template <int NCH>
__device__ __forceinline__ uint32_t scale_pair(const u32x4* sv, const uint32_t* s2, int c) {
  if constexpr (NCH % 8 == 0) {
    const uint32_t w = sv[c / 8][(c % 8) / 2];
    return (c & 1) ? (w >> 16) : (w & 0xFFFFu);
  } else {
    return s2[c];
  }
}

template <int NCH, int WPB>
__global__ __launch_bounds__(64 * WPB) void k_dec_gate_up(
    const uint8_t* __restrict__ gu_codes, const uint8_t* __restrict__ gu_scales,
    const float* __restrict__ scale2, const _Float16* __restrict__ xh,
    const float* __restrict__ unmul, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slot, const int32_t* __restrict__ groups, int T, int K,
    int H, int I, int has_shared, uint16_t* __restrict__ h) {
  extern __shared__ __align__(16) _Float16 xl[];  // [T][H + 8] f16
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, r16 = lane & 15, q = lane >> 4;
  const int ld = H + 8, Q = H / 4;
  const int nbk = I / 16 / WPB;
  const int a = blockIdx.x / nbk, pb = (blockIdx.x % nbk) * WPB + wv;

  // activation rows into LDS: loads issued before anything that depends on the group
  {
    const int chunks = T * (H / 8);
    for (int c = threadIdx.x; c < chunks; c += 64 * WPB) {
      const int r = c / (H / 8), ch = c % (H / 8);
      *(u32x4*)(xl + (size_t)r * ld + 8 * ch) = *(const u32x4*)(xh + (size_t)r * H + 8 * ch);
    }
  }
  float um[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) um[i] = (4 * q + i < T) ? unmul[4 * q + i] : 0.f;

  const bool active = a < groups[0];
  int e = 0;
  GURegs<NCH> w;
  if (active) {
    e = groups[1 + a];
    const size_t rowb = (size_t)H / 2, srow = (size_t)H / 16;
    const size_t grow = (size_t)e * 2 * I + (size_t)pb * 16 + r16;
    const uint8_t* cg = gu_codes + grow * rowb + (size_t)(Q / 2) * q;
    const uint8_t* cu = cg + (size_t)I * rowb;
    const uint8_t* sg = gu_scales + grow * srow + (size_t)(Q / 16) * q;
    const uint8_t* su = sg + (size_t)I * srow;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      w.g[c] = *(const u32x4*)(cg + 16 * c);
      w.u[c] = *(const u32x4*)(cu + 16 * c);
    }
    if constexpr (NCH % 8 == 0) {
#pragma unroll
      for (int c = 0; c < NCH / 8; ++c) {
        w.sg[c] = *(const u32x4*)(sg + 16 * c);
        w.su[c] = *(const u32x4*)(su + 16 * c);
      }
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        w.sg2[c] = *(const uint16_t*)(sg + 2 * c);
        w.su2[c] = *(const uint16_t*)(su + 2 * c);
      }
    }
  }
  __syncthreads();  // activations in LDS
  if (!active) return;
  const int p0 = offsets[e], n = offsets[e + 1] - p0;
  const float s2g = scale2[3 * e + 0], s2u = scale2[3 * e + 1];
  const int tokl = (lane < n) ? slot_token(sorted_slot[p0 + lane], T, K, has_shared) : -1;

  f32x4 dg = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
  const _Float16* xr = xl + (size_t)r16 * ld + Q * q;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const f16x2 sgv = e4m3x2_to_f16(scale_pair<NCH>(w.sg, w.sg2, c));
    const f16x2 suv = e4m3x2_to_f16(scale_pair<NCH>(w.su, w.su2, c));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x8 av = __builtin_bit_cast(f16x8, u32x4{0u, 0u, 0u, 0u});
      if (r16 < T) av = *(const f16x8*)(xr + 32 * c + 8 * j);
      dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(w.g[c][j], j < 2 ? sgv.x : sgv.y), dg, 0, 0, 0);
      du = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dqh8(w.u[c][j], j < 2 ? suv.x : suv.y), du, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  uint16_t hv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float g = dg[i] * um[i] * s2g, u = du[i] * um[i] * s2u;
    hv[i] = f32_to_bf16_bits(silu_f32(g) * u);
  }
  // position p of the group holds token tok(p); lane (tok/4, col) has its row
  const int j = pb * 16 + r16;
  for (int p = 0; p < n; ++p) {
    const int tok = p < 64 ? __shfl(tokl, p, 64) : slot_token(sorted_slot[p0 + p], T, K, has_shared);
    if (tok >= 0 && (tok >> 2) == q) {
      const int i = tok & 3;
      h[(size_t)(p0 + p) * I + j] = i == 0 ? hv[0] : (i == 1 ? hv[1] : (i == 2 ? hv[2] : hv[3]));
    }
  }
}

// --------------------------------- down -----------------------------------
// One wave = one unit (group, 64 output rows as 4 MFMA blocks of 16, all of
// K = I); a block holds WPB consecutive units of one group and the group's h
// rows (up to 16 per pass) in LDS.  Lane (r16, q) owns K elements
// [Q*q, Q*q + Q), Q = I/4, as 16-byte code chunks; its Q/16 scale bytes are
// contiguous.

template <int NCH>   // NCH = I / 128
struct DNRegs {
  u32x4 c[4][NCH];
  uint32_t s[4][NCH];  // 2 scale bytes per chunk, in the low half
};

template <int NCH, int WPB>
__global__ __launch_bounds__(64 * WPB) void k_dec_down(
    const uint8_t* __restrict__ dn_codes, const uint8_t* __restrict__ dn_scales,
    const float* __restrict__ scale2, const uint16_t* __restrict__ h,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ groups, int T, int K, int H, int I, int has_shared,
    uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) uint16_t hl[];  // [16][I + 8]: h rows of one pass
  __shared__ int rvl[16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, r16 = lane & 15, q = lane >> 4;
  const int Q = I / 4, ldh = I + 8;
  const int nbk = H / 64 / WPB;
  const int a = blockIdx.x / nbk, rb = (blockIdx.x % nbk) * WPB + wv;
  if (a >= groups[0]) return;  // uniform per block
  const int e = groups[1 + a];
  const size_t rowb = (size_t)I / 2, srow = (size_t)I / 16;
  DNRegs<NCH> w;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const size_t row = (size_t)e * H + (size_t)rb * 64 + nb * 16 + r16;
    const uint8_t* cr = dn_codes + row * rowb + (size_t)(Q / 2) * q;
    const uint8_t* sr = dn_scales + row * srow + (size_t)(Q / 16) * q;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      w.c[nb][c] = *(const u32x4*)(cr + 16 * c);
      w.s[nb][c] = *(const uint16_t*)(sr + 2 * c);
    }
  }
  const int p0 = offsets[e], n = offsets[e + 1] - p0;
  const float s2d = scale2[3 * e + 2];
  for (int r0 = 0; r0 < n; r0 += 16) {  // one pass unless ids repeat (> 16 rows)
    if (r0 > 0) __syncthreads();          // previous pass done reading hl
    for (int c = threadIdx.x; c < 16 * (I / 8); c += 64 * WPB) {
      const int r = c / (I / 8), ch = c % (I / 8);
      const int m = r0 + r;
      const bool rv = m < n && slot_token(sorted_slot[p0 + m], T, K, has_shared) >= 0;
      *(u32x4*)(&hl[r * ldh + 8 * ch]) = rv ? *(const u32x4*)(h + (size_t)(p0 + m) * I + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
      if (ch == 0) rvl[r] = rv ? 1 : 0;
    }
    __syncthreads();
    // the weight words count as redefined on every pass, so the dequantised
    // operands (4x the registers of the codes) are not hoisted out of the loop
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int c = 0; c < NCH; ++c) asm volatile("" : "+v"(w.c[nb][c]));
    f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float sc[4][2];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        sc[nb][0] = e4m3_to_f32(w.s[nb][c] & 0xFFu);
        sc[nb][1] = e4m3_to_f32((w.s[nb][c] >> 8) & 0xFFu);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4*)(&hl[r16 * ldh + Q * q + 32 * c + 8 * j]));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, dq8(w.c[nb][c][j], sc[nb][j >> 1]), acc[nb], 0, 0, 0);
      }
      // keep each chunk's dequantised operands next to their MFMAs (bounds
      // the registers in flight)
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int col = rb * 64 + nb * 16 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mm = 4 * q + i;
        if (r0 + mm < n && rvl[mm]) y[(size_t)(p0 + r0 + mm) * H + col] = f32_to_bf16_bits(acc[nb][i] * s2d);
      }
    }
  }
}

// --------------------------------- host -----------------------------------

void register_decode_kernels(std::vector<const void*>& k) {
  k.push_back((const void*)&k_dec_xprep<false>);
  k.push_back((const void*)&k_dec_xprep<true>);
  k.push_back((const void*)&k_dec_gate_up<2, 1>);
  k.push_back((const void*)&k_dec_gate_up<2, 4>);
  k.push_back((const void*)&k_dec_gate_up<4, 1>);
  k.push_back((const void*)&k_dec_gate_up<4, 4>);
  k.push_back((const void*)&k_dec_gate_up<8, 1>);
  k.push_back((const void*)&k_dec_gate_up<8, 4>);
  k.push_back((const void*)&k_dec_gate_up<16, 1>);
  k.push_back((const void*)&k_dec_gate_up<16, 4>);
  k.push_back((const void*)&k_dec_down<1, 1>);
  k.push_back((const void*)&k_dec_down<1, 4>);
  k.push_back((const void*)&k_dec_down<2, 1>);
  k.push_back((const void*)&k_dec_down<2, 4>);
  k.push_back((const void*)&k_dec_down<4, 1>);
  k.push_back((const void*)&k_dec_down<4, 4>);
  k.push_back((const void*)&k_dec_down<8, 1>);
  k.push_back((const void*)&k_dec_down<8, 4>);
}

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Shapes the decode kernels are instantiated for (others take the grouped path).
bool decode_supported(int H, int I) {
  const int nch = H / 128, ncd = I / 128;
  return (nch == 2 || nch == 4 || nch == 8 || nch == 16) &&
         (ncd == 1 || ncd == 2 || ncd == 4 || ncd == 8);
}

// f16 activation rows [T][H] and their epilogue factors [T].
size_t decode_workspace_extra(int T, int H) {
  return align256((size_t)T * H * sizeof(_Float16)) + align256((size_t)T * sizeof(float));
}

hipError_t launch_decode_ffn(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                             const int32_t* offsets, const int32_t* sorted_slot,
                             const int32_t* groups, bool fp8, uint16_t* hbuf, uint8_t* xq,
                             float* xs, void* dec_ws, uint16_t* y, hipStream_t s) {
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const int G = W.E + hs;
  const int gmax = (int)((long)T * K + hs < (long)G ? (long)T * K + hs : (long)G);
  _Float16* xh = (_Float16*)dec_ws;
  float* unmul = (float*)((uint8_t*)dec_ws + align256((size_t)T * H * sizeof(_Float16)));
  const dim3 blk(256);
  if (fp8)
    MOE_LAUNCH("dec_xprep", s, (k_dec_xprep<true>), dim3(T), blk, 0, s, x, H, xh, unmul, xq, xs);
  else
    MOE_LAUNCH("dec_xprep", s, (k_dec_xprep<false>), dim3(T), blk, 0, s, x, H, xh, unmul, xq, xs);
  // Waves (units) per block: 4 when there are enough units to fill the
  // chip, else 1 so that small T still spreads over many CUs.
  const long gu_units = (long)gmax * (I / 16), dn_units = (long)gmax * (H / 64);
  const long cus = num_cus();
  const int wpb_g = gu_units >= 8 * cus ? 4 : 1;
  const int wpb_d = dn_units >= 8 * cus ? 4 : 1;
  const size_t lds_gu = (size_t)T * (H + 8) * sizeof(_Float16);
  const dim3 g1((unsigned)(gu_units / wpb_g)), b1(64 * wpb_g);
  const int nch = H / 128;
#define MOE_DEC_GU(NCH)                                                                             \
  do {                                                                                              \
    if (wpb_g == 4)                                                                                 \
      MOE_LAUNCH("dec_gate_up", s, (k_dec_gate_up<NCH, 4>), g1, b1, lds_gu, s, W.gu_codes,          \
                 W.gu_scales, W.scale2, xh, unmul, offsets, sorted_slot, groups, T, K, H, I, hs, hbuf); \
    else                                                                                            \
      MOE_LAUNCH("dec_gate_up", s, (k_dec_gate_up<NCH, 1>), g1, b1, lds_gu, s, W.gu_codes,          \
                 W.gu_scales, W.scale2, xh, unmul, offsets, sorted_slot, groups, T, K, H, I, hs, hbuf); \
  } while (0)
  if (nch == 2) MOE_DEC_GU(2);
  else if (nch == 4) MOE_DEC_GU(4);
  else if (nch == 8) MOE_DEC_GU(8);
  else if (nch == 16) MOE_DEC_GU(16);
  else return hipErrorInvalidValue;
#undef MOE_DEC_GU
  const dim3 g2((unsigned)(dn_units / wpb_d)), b2(64 * wpb_d);
  const size_t lds_dn = (size_t)16 * (I + 8) * sizeof(uint16_t);
  const int ncd = I / 128;
#define MOE_DEC_DN(NCH)                                                                            \
  do {                                                                                             \
    if (wpb_d == 4)                                                                                \
      MOE_LAUNCH("dec_down", s, (k_dec_down<NCH, 4>), g2, b2, lds_dn, s, W.dn_codes, W.dn_scales,       \
                 W.scale2, hbuf, offsets, sorted_slot, groups, T, K, H, I, hs, y);                 \
    else                                                                                           \
      MOE_LAUNCH("dec_down", s, (k_dec_down<NCH, 1>), g2, b2, lds_dn, s, W.dn_codes, W.dn_scales,       \
                 W.scale2, hbuf, offsets, sorted_slot, groups, T, K, H, I, hs, y);                 \
  } while (0)
  if (ncd == 1) MOE_DEC_DN(1);
  else if (ncd == 2) MOE_DEC_DN(2);
  else if (ncd == 4) MOE_DEC_DN(4);
  else if (ncd == 8) MOE_DEC_DN(8);
  else return hipErrorInvalidValue;
#undef MOE_DEC_DN
  return hipGetLastError();
}

}  // namespace moe
