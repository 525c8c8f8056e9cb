// Router gating GEMM fused with the top-K (the router stage of the layer):
// logits = x . W_r^T with an NVFP4 router matrix (e2m1 codes, one e4m3 scale
// per 16 K, one fp32 scale2) against the bf16 activation rows, then the top-K
// of each token's logits in the same block, plus the shared-expert gate logit
// when the matrix has a gate row (index E).  The pages list the router GEMM
// and top-k as the first prefill op that changes the logits (issue "[job]
// Qwen3.8-Flash-Next: long-context cold prefill to SGLang parity", section
// "Localising the remaining ~0.56 %") and profile it as a w4a16 GEMM (same
// issue, the nsys kernel table).
//
// A block takes 16 tokens and all E experts (padded to 64 NBW per 4 waves).
// Wave w owns NBW n-blocks of 16 router rows: MFMA 16x16x32 bf16 with the
// dequantised router rows as the A operand (lane (n = l%16, q = l/16) loads
// bytes [64c + 16q, +16) of row n's 128-byte K-step slice, c = 0, 1; MFMA k
// index 8q + i is element 128c + 32q + 8jj + i of the step) and the token
// rows as the B operand, f32 accumulation; the lane holding token column t
// gets 4 consecutive experts of it.  The K loop prefetches half a step ahead
// (chunk 0 of step s + 1 while chunk 1 of step s computes).  Every load is a
// buffer load with a range check, so rows >= E read zeros.
//
// The fp32 logits (times scale2) go to LDS [16][E_pad]; the gate row's logit
// is a fixed-order wave sum of exact products; then each wave routes its
// tokens with route_row_topk (moe_topk.hpp) straight from LDS, and the logits
// are copied out when the caller asks for them.
#include "moe_ffn_common.hpp"
#include "moe_internal.hpp"
#include "moe_topk.hpp"

namespace moe {

namespace {

constexpr int kRK = 256;  // K elements per step
constexpr int kBufferFlags = 0x00020000;

template <int NBW, int WPB>
__global__ __launch_bounds__(64 * WPB) void k_router_topk(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, float scale2,
    const uint16_t* __restrict__ x, int T, int E, int K, int H, int has_gate,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ logits,
    float* __restrict__ gate) {
  constexpr int EP = 16 * NBW * WPB;  // padded experts
  extern __shared__ __align__(16) float zl[];  // [16][EP]
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m16 = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 16;
  const uint32_t rowb = (uint32_t)H / 2, srow = (uint32_t)H / 16;
  const int nsteps = H / kRK;

  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)codes, (short)0, (int)((uint32_t)E * rowb), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)scales, (short)0, (int)((uint32_t)E * srow), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, (short)0, (int)((uint32_t)T * (uint32_t)H * 2u), kBufferFlags);
  const int row0 = 16 * NBW * wv + m16;                 // the lane's router row in n-block 0
  const uint32_t wlane = (uint32_t)row0 * rowb + 16u * q;
  const uint32_t slane = (uint32_t)row0 * srow + 2u * q;
  const int tok = min(t0 + m16, T - 1);                 // padding tokens read the last row
  const uint32_t xlane = (uint32_t)tok * (uint32_t)H * 2u + 64u * q;

  u32x4 wc[2][NBW], xc[2][4];
  uint32_t sc[2][NBW];
  auto load = [&](int c, int s) {  // chunk c of step s
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      // the whole offset in the range-checked voffset: padded rows (>= E) read 0
      wc[c][nb] = __builtin_amdgcn_raw_buffer_load_b128(
          rw, (int)(wlane + 64u * c + 128u * s + (uint32_t)nb * 16u * rowb), 0, 0);
      sc[c][nb] = __builtin_amdgcn_raw_buffer_load_b16(
          rs, (int)(slane + 8u * c + 16u * s + (uint32_t)nb * 16u * srow), 0, 0);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      xc[c][jj] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)xlane + 256 * c + 16 * jj,
                                                        2 * kRK * s, 0);
  };
  f32x4 acc[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int c) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc[c][nb], 1.0f, false);
        const bf16x8 a = dq8(wc[c][nb][jj], jj < 2 ? sv.x : sv.y);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, xc[c][jj]),
                                                          acc[nb], 0, 0, 0);
      }
    }
  };
  load(0, 0);
  load(1, 0);
  for (int s = 0; s < nsteps; ++s) {
    compute(0);
    if (s + 1 < nsteps) load(0, s + 1);
    compute(1);
    if (s + 1 < nsteps) load(1, s + 1);
  }
  // logits -> LDS: lane (t, g) holds experts 16 nb + 4 g + [0, 4) of its
  // wave's rows for token t
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const f32x4 v = acc[nb] * scale2;
    *(f32x4*)&zl[m16 * EP + 16 * NBW * wv + 16 * nb + 4 * q] = v;
  }
  // the shared-expert gate logit: row E, a fixed-order wave sum of exact
  // products (8 consecutive K elements per lane per pass)
  if (has_gate) {
    const uint8_t* gc = codes + (size_t)E * rowb;
    const uint8_t* gs = scales + (size_t)E * srow;
    for (int t = wv; t < 16; t += WPB) {
      if (t0 + t >= T) break;  // uniform per wave
      const uint16_t* xr = x + (size_t)(t0 + t) * H;
      float part = 0.f;
      for (int k0 = 8 * lane; k0 < H; k0 += 512) {
        const uint32_t cw = *(const uint32_t*)(gc + k0 / 2);
        const f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)gs[k0 / 16], 1.0f, false);
        const float s8 = sv.x;
        const u32x4 xv = *(const u32x4*)(xr + k0);
        const f32x2 wps[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0),
                              __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1),
                              __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2),
                              __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3)};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const f32x2 wp = wps[p];
          part = fmaf(wp.x * s8, bf16_bits_to_f32(xv[p] & 0xFFFFu), part);
          part = fmaf(wp.y * s8, bf16_bits_to_f32(xv[p] >> 16), part);
        }
      }
      const float g = wave_sum_dpp(part) * scale2;
      if (lane == 0) gate[t0 + t] = g;
    }
  }
  __syncthreads();
  for (int t = wv; t < 16; t += WPB) {
    if (t0 + t >= T) break;  // uniform per wave
    const size_t tt = (size_t)(t0 + t);
    route_row_topk<NBW * WPB / 4>(&zl[t * EP], E, K, ids + tt * K, w + tt * K);
    if (logits)
      for (int e = lane; e < E; e += 64) logits[tt * E + e] = zl[t * EP + e];
  }
}

}  // namespace

void register_router_kernels(std::vector<const void*>& k) {
  k.push_back((const void*)&k_router_topk<1, 4>);
  k.push_back((const void*)&k_router_topk<2, 4>);
  k.push_back((const void*)&k_router_topk<4, 4>);
  k.push_back((const void*)&k_router_topk<8, 4>);
  k.push_back((const void*)&k_router_topk<8, 8>);
}

hipError_t launch_router_topk(const moe_nvfp4_router& R, const uint16_t* x, int T, int K,
                              int32_t* ids, float* w, float* logits, float* gate,
                              hipStream_t s) {
  const int E = R.E, H = R.H;
  const dim3 grid((unsigned)((T + 15) / 16));
#define MOE_ROUTER(NBW, WPB)                                                                    \
  MOE_LAUNCH("router_topk", s, (k_router_topk<NBW, WPB>), grid, dim3(64 * WPB),                 \
             (size_t)16 * 16 * NBW * WPB * sizeof(float), s, R.codes, R.scales, R.scale2, x, T, \
             E, K, H, R.has_gate, ids, w, logits, gate)
  if (E <= 64) MOE_ROUTER(1, 4);
  else if (E <= 128) MOE_ROUTER(2, 4);
  else if (E <= 256) MOE_ROUTER(4, 4);
  else if (E <= 512) MOE_ROUTER(8, 4);
  else MOE_ROUTER(8, 8);
#undef MOE_ROUTER
  return hipGetLastError();
}

}  // namespace moe
