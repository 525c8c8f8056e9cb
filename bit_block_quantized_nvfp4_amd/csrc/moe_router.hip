// Router gating GEMM: logits = scale2 * x . W_r^T with an NVFP4 router matrix
// (e2m1 codes, one e4m3 scale per 16 K, one fp32 scale2) against the bf16
// activation rows, followed by the router's top-K on those logits.  The pages
// list the router GEMM and its top-k as the first prefill op that changes the
// logits (issue "[job] Qwen3.8-Flash-Next: long-context cold prefill to
// SGLang parity", section "Localising the remaining ~0.56 %") and profile the
// router as a w4a16 GEMM (same issue, the nsys kernel table).
//
// Both GEMM kernels use MFMA 16x16x32 bf16 with the dequantised router rows as
// the A operand and the token rows as the B operand.  For 16 rows n and a
// K step of 256, lane (n = l%16, q = l/16) loads bytes [64c + 16q, +16) of row
// n's 128-byte slice (chunk c = 0, 1): MFMA jj of chunk c takes K elements
// 128c + 32q + 8jj + [0, 8) of the step on both operands.  The accumulator of
// lane (t, q) holds rows 4q + [0, 4) for token column t.  Every weight load is
// a range-checked buffer load with the whole offset in the voffset, so rows
// past the matrix read zeros.
//
// * k_router_splitk (T <= kSplitMaxT): a block takes 16 tokens x 16 router
//   rows (the gate row E included) and its 4 waves split K (wave w takes steps
//   w, w + 4, ...), all loads of a wave in flight together, so the latency is
//   about one memory round trip.  The 4 partial sums are added in wave order
//   through LDS.
// * k_router_tiled (larger T): a block takes 16*TB tokens x 64*NB experts; the
//   token rows of each K step are staged in LDS by direct buffer->LDS loads
//   (double buffered, 16-byte columns XOR-swizzled by row so the B reads are
//   free of bank conflicts) and each dequantised weight operand feeds TB
//   MFMAs, which keeps the NVFP4 dequant (16 VALU operations per 8 weights,
//   the conversions among them slower than plain VALU) from bounding the
//   kernel.  The e4m3 scales go through LDS as whole 128-byte row pieces:
//   a load instruction whose 64 lanes touch 16 rows (16 cache lines) costs
//   several times one that reads 1 KB contiguous, so the per-lane 2-byte
//   scale loads would cost as much as the code loads.  The gate row is a VALU
//   dot product over the same staged rows (blocks of the first expert tile),
//   a fixed-order sum.
//
// The top-K is the router stage's own kernel (moe_route.hip) on the logits.
#include "moe_ffn_common.hpp"
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int kBufferFlags = 0x00020000;
constexpr int kSplitMaxT = 1024;  // largest T routed through the split-K kernel

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, kBufferFlags);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float e4m3_lo(uint32_t b) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b, 1.0f, false);
  return v.x;
}

// ---------------------------------------------------------------- split-K
__global__ __launch_bounds__(256) void k_router_splitk(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, float scale2,
    const uint16_t* __restrict__ x, int T, int E, int R, int H, float* __restrict__ logits,
    float* __restrict__ gate) {
  __shared__ f32x4 part[4][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 16, r0 = blockIdx.y * 16;
  const uint32_t rowb = (uint32_t)H / 2, srow = (uint32_t)H / 16;
  const int nsteps = H / 256;
  const __amdgpu_buffer_rsrc_t rw = rsrc(codes, (uint32_t)R * rowb);
  const __amdgpu_buffer_rsrc_t rs = rsrc(scales, (uint32_t)R * srow);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint32_t)T * (uint32_t)H * 2u);
  const uint32_t wlane = (uint32_t)(r0 + n) * rowb + 16u * q;
  const uint32_t slane = (uint32_t)(r0 + n) * srow + 2u * q;
  const uint32_t xlane = (uint32_t)min(t0 + n, T - 1) * (uint32_t)H * 2u + 64u * q;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // two steps (s and s + 4) per pass, all of their loads issued together
  for (int s = wv; s < nsteps; s += 8) {
    const bool two = s + 4 < nsteps;  // wave-uniform
    const int s1 = two ? s + 4 : s;
    u32x4 wc[2][2], xc[2][2][4];
    uint32_t sc[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t ss = (uint32_t)(h ? s1 : s);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        wc[h][c] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(wlane + 128u * ss + 64u * c), 0, 0);
        sc[h][c] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(slane + 16u * ss + 8u * c), 0, 0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          xc[h][c][jj] = __builtin_amdgcn_raw_buffer_load_b128(
              rx, (int)(xlane + 512u * ss + 256u * c + 16u * jj), 0, 0);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1 && !two) break;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc[h][c], 1.0f, false);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8(wc[h][c][jj], jj < 2 ? sv.x : sv.y),
                                                        __builtin_bit_cast(bf16x8, xc[h][c][jj]),
                                                        acc, 0, 0, 0);
      }
    }
  }
  part[wv][lane] = acc;
  __syncthreads();
  // thread (token t, row rr): the four wave partials in wave order
  const int t = threadIdx.x >> 4, rr = threadIdx.x & 15;
  const int src = t + 16 * (rr >> 2), v = rr & 3;
  const float z = (((part[0][src][v] + part[1][src][v]) + part[2][src][v]) + part[3][src][v]) * scale2;
  const int tok = t0 + t, row = r0 + rr;
  if (tok < T) {
    if (row < E) logits[(size_t)tok * E + row] = z;
    else if (row == E && gate) gate[tok] = z;
  }
}

// ------------------------------------------------------------------ tiled
// The block's e4m3 scales sit in LDS, a [16 NB x 4 rows][128 B] tile per
// 2048 K (8 steps; two tiles when H > 2048), loaded as whole 128-byte row
// pieces (8 rows per 1 KB DMA instruction) with piece p of row r at slot
// p ^ (r & 7), so the per-lane 2-byte scale reads spread over the banks; the
// codes go straight to registers.
template <int TB, int NB>
__global__ __launch_bounds__(256) void k_router_tiled(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, float scale2,
    const uint16_t* __restrict__ x, int T, int E, int H, int has_gate,
    float* __restrict__ logits, float* __restrict__ gate) {
  constexpr int TT = 16 * TB;      // tokens per block
  constexpr int ET = 64 * NB;      // experts per block (4 waves)
  constexpr int XS = TT * 512;     // bytes of one staged K step (TT rows x 256 bf16)
  constexpr int SS = ET * 128;     // bytes of one scale tile (8 steps)
  constexpr int GP = 256 / TT;     // gate: threads per token
  constexpr int GK = 256 / GP;     // gate: K elements per thread per step
  extern __shared__ __align__(16) uint8_t xs[];  // [2][XS] x stages, then 1 or 2 scale tiles
  uint8_t* const ss = xs + 2 * XS;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * TT;
  const int e0 = blockIdx.y * ET;
  const uint32_t rowb = (uint32_t)H / 2, srow = (uint32_t)H / 16;
  const int nsteps = H / 256;
  const __amdgpu_buffer_rsrc_t rw = rsrc(codes, (uint32_t)E * rowb);
  const __amdgpu_buffer_rsrc_t rs = rsrc(scales, (uint32_t)E * srow);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint32_t)T * (uint32_t)H * 2u);
  const uint32_t wrow = (uint32_t)(e0 + 16 * NB * wv + n);
  const uint32_t wlane = wrow * rowb + 16u * q;

  // x stage: 1 KB per wave instruction = two token rows; LDS column p of row r
  // holds source column p ^ (r & 15)
  auto load_x = [&](int st, int s) {
#pragma unroll
    for (int i = 0; i < 2 * TB; ++i) {
      const int blk = wv * 2 * TB + i;
      const int row = 2 * blk + (lane >> 5);
      const int col = (lane & 31) ^ (row & 15);
      const uint32_t tok = (uint32_t)min(t0 + row, T - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)&xs[st * XS + 1024 * blk], 16,
                                               (int)(tok * (uint32_t)H * 2u + 16u * col),
                                               512 * s, 0, 0);
    }
  };
  // scale tile kc (steps 8 kc ..): wave wv loads its 16 NB rows, 8 per
  // instruction; lane L writes slot L & 7 of row L >> 3 (mod 8), i.e. piece
  // (L & 7) ^ (L >> 3)
  auto load_s = [&](int sb, int kc) {
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) {
      const uint32_t r = (uint32_t)(16 * NB * wv + 8 * i + (lane >> 3));
      const uint32_t piece = (uint32_t)((lane & 7) ^ (lane >> 3));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_ptr_t)&ss[sb * SS + 2048 * NB * wv + 1024 * i], 16,
          (int)((e0 + r) * srow + 128u * kc + 16u * piece), 0, 0, 0);
    }
  };
  u32x4 wc[2][NB];
  auto load_w = [&](int c, int s) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      wc[c][nb] = __builtin_amdgcn_raw_buffer_load_b128(
          rw, (int)(wlane + (uint32_t)nb * 16u * rowb + 128u * s + 64u * c), 0, 0);
  };
  f32x4 acc[NB][TB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[nb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int c, int st, int s) {
    // row 16 NB wv + 16 nb + n: its piece s & 7 sits at slot (s & 7) ^ (n & 7)
    const uint8_t* srw = &ss[((s >> 3) & 1) * SS + (16 * NB * wv + n) * 128 +
                             16 * ((s & 7) ^ (n & 7)) + 8 * c + 2 * q];
    float sv[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(
          (uint32_t) * (const uint16_t*)(srw + 16 * 128 * nb), 1.0f, false);
      sv[nb][0] = v.x;
      sv[nb][1] = v.y;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      bf16x8 b[TB];
      const int colp = (16 * c + 4 * q + jj) ^ n;  // row & 15 == n for row 16 tb + n
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        b[tb] = *(const bf16x8*)&xs[st * XS + (16 * tb + n) * 512 + 16 * colp];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 a = dq8(wc[c][nb][jj], sv[nb][jj >> 1]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          acc[nb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[tb], acc[nb][tb], 0, 0, 0);
      }
    }
  };

  // gate row: thread (token gt, part gp) takes K elements [GK gp, GK gp + GK)
  // of each step
  const bool gate_blk = has_gate && blockIdx.y == 0;  // block-uniform
  const int gt = threadIdx.x / GP, gp = threadIdx.x % GP;
  const uint8_t* gcodes = codes + (size_t)E * rowb + (size_t)(GK / 2) * gp;
  const uint8_t* gscales = scales + (size_t)E * srow + (size_t)(GK / 16) * gp;
  float gacc = 0.f;

  load_s(0, 0);
  load_x(0, 0);
  load_w(0, 0);
  load_w(1, 0);
  wait_vmcnt<0>();
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int st = s & 1;
    const int sn = min(s + 1, nsteps - 1);  // the last step reloads itself (unused)
    uint32_t gc[GK / 8];  // 8 codes per word
    uint32_t gs = 0;      // GK / 16 scale bytes
    if (gate_blk) {
#pragma unroll
      for (int j = 0; j < GK / 8; ++j) gc[j] = *(const uint32_t*)(gcodes + 128 * s + 4 * j);
      gs = (GK == 64)   ? *(const uint32_t*)(gscales + 16 * s)
           : (GK == 32) ? (uint32_t) * (const uint16_t*)(gscales + 16 * s)
                        : (uint32_t)gscales[16 * s];
    }
    if ((sn & 7) == 0 && sn != s) load_s((sn >> 3) & 1, sn >> 3);  // next scale tile
    load_x(st ^ 1, sn);
    compute(0, st, s);
    load_w(0, sn);
    compute(1, st, s);
    load_w(1, sn);
    if (gate_blk) {
      const int gr = gt & 15;
#pragma unroll
      for (int j = 0; j < GK / 8; ++j) {
        const uint32_t cw = gc[j];
        const float s8 = e4m3_lo(gs >> (8 * (j / 2)));
        const int colp = ((GK / 8) * gp + j) ^ gr;
        const u32x4 xv = *(const u32x4*)&xs[st * XS + gt * 512 + 16 * colp];
        const f32x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
        const f32x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
        const f32x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
        const f32x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
        gacc = fmaf(w0.x * s8, bf16_bits_to_f32(xv[0] & 0xFFFFu), gacc);
        gacc = fmaf(w0.y * s8, bf16_bits_to_f32(xv[0] >> 16), gacc);
        gacc = fmaf(w1.x * s8, bf16_bits_to_f32(xv[1] & 0xFFFFu), gacc);
        gacc = fmaf(w1.y * s8, bf16_bits_to_f32(xv[1] >> 16), gacc);
        gacc = fmaf(w2.x * s8, bf16_bits_to_f32(xv[2] & 0xFFFFu), gacc);
        gacc = fmaf(w2.y * s8, bf16_bits_to_f32(xv[2] >> 16), gacc);
        gacc = fmaf(w3.x * s8, bf16_bits_to_f32(xv[3] & 0xFFFFu), gacc);
        gacc = fmaf(w3.y * s8, bf16_bits_to_f32(xv[3] >> 16), gacc);
      }
    }
    wait_vmcnt<2 * NB>();  // everything but the 2 x NB code loads: x and scales landed
    __syncthreads();
  }
  wait_vmcnt<0>();

  if (gate_blk) {
    // the GP partials of a token sit in consecutive lanes: butterfly, fixed order
#pragma unroll
    for (int m = 1; m < GP; m <<= 1) gacc += __shfl_xor(gacc, m);
    if (gp == 0 && t0 + gt < T) gate[t0 + gt] = gacc * scale2;
  }
  const bool vec = (E & 3) == 0;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = e0 + 16 * NB * wv + 16 * nb + 4 * q;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int tok = t0 + 16 * tb + n;
      if (tok >= T || e >= E) continue;
      const f32x4 z = acc[nb][tb] * scale2;
      float* dst = logits + (size_t)tok * E + e;
      if (vec && e + 4 <= E) {
        *(f32x4*)dst = z;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (e + v < E) dst[v] = z[v];
      }
    }
  }
}

}  // namespace

void register_router_kernels(std::vector<const void*>& k) {
  k.push_back((const void*)&k_router_splitk);
  k.push_back((const void*)&k_router_tiled<2, 2>);
  k.push_back((const void*)&k_router_tiled<4, 2>);
}

hipError_t launch_router_topk(const moe_nvfp4_router& R, const uint16_t* x, int T, int K,
                              int32_t* ids, float* w, float* logits, float* gate,
                              hipStream_t s) {
  const int E = R.E, H = R.H;
  if (T <= kSplitMaxT) {
    const int rows = E + (R.has_gate ? 1 : 0);
    const dim3 grid((unsigned)((T + 15) / 16), (unsigned)((rows + 15) / 16));
    MOE_LAUNCH("router_gemm", s, k_router_splitk, grid, dim3(256), 0, s, R.codes, R.scales,
               R.scale2, x, T, E, rows, H, logits, gate);
  } else {
    const int tiles = H > 2048 ? 2 : 1;  // scale tiles held at once
#define MOE_ROUTER_TILED(TB, NB)                                                                 \
  MOE_LAUNCH("router_gemm", s, (k_router_tiled<TB, NB>),                                        \
             dim3((unsigned)((T + 16 * TB - 1) / (16 * TB)), (unsigned)((E + 64 * NB - 1) / (64 * NB))), \
             dim3(256), (size_t)(2 * 16 * TB * 512 + tiles * 64 * NB * 128), s, R.codes, R.scales, \
             R.scale2, x, T, E, H, R.has_gate, logits, gate)
    if (T <= 8192) MOE_ROUTER_TILED(2, 2);
    else MOE_ROUTER_TILED(4, 2);
#undef MOE_ROUTER_TILED
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_route_topk(logits, T, E, K, ids, w, s);
}

}  // namespace moe
