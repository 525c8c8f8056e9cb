// Fused prefill expert FFN: gate_up GEMM -> SiLU * up -> down GEMM of one
// work item = (group, 128-row tile of its sorted rows) in one block, one
// launch for the whole layer (T > 8 tokens; H % 512 == 0, I % 512 == 0).
//
//   gate_up: A = f16 activation rows gathered by token (x with a per-row
//            power-of-two shift, or the exact f16 value of the FP8 arm's e4m3
//            codes), B = NVFP4 gate/up rows dequantised to f16 (one
//            instruction per element), f32 accumulate; epilogue
//            h = bf16(silu(g * s2g * f_t) * (u * s2u * f_t)), f_t the row's
//            epilogue factor, stored to the workspace by sorted position;
//   down:    A = those bf16 h rows, read straight back by the same block (they
//            are still in L2).  At I = 512 the whole h tile stays in LDS for
//            all N tiles and is turned into f16 in place with a per-row power
//            of two (undone in the epilogue), B = NVFP4 down rows dequantised
//            to f16; otherwise A streams as bf16 and B is dequantised to bf16.
//            Epilogue y = bf16(acc * f_r * s2d).
//
// MFMA 16x16x32 (f16 for gate_up, bf16 for down).  A block of 8 waves (two
// per SIMD, so one wave's LDS, dequant and barrier waits overlap the other's
// MFMAs) owns an N tile of 512 weight rows: wave w holds 4 n-blocks of 16
// rows (gate_up: 32 gate rows and the 32 up rows of the same pairs, so g and
// u of one pair sit in the same lane) against every valid 16-row m-block of
// the tile.
//
// K runs in steps of 256 elements.  Weight codes go straight from global
// memory into each wave's registers (only the owning wave reads them): lane
// (n = l%16, q = l/16) loads bytes [64c + 16q, +16) of its row's 128-byte step
// slice for c = 0, 1, so each load instruction covers 64 contiguous bytes of
// 16 rows, and both halves of every 128-byte line are requested within the
// same step.  The step's A tile
// (valid rows x 512 B) and block scales (512 rows x 16 B) go to a
// double-buffered LDS stage by global->LDS DMA; everything for step s+1 is
// issued before step s computes; one wait and one barrier per step.  A rows
// are XOR-swizzled in 16-byte chunks so the operand reads of 16 rows at one
// chunk hit 16 distinct bank groups.
//
// Lane (n, q) of sub-MFMA (c, jj), c in {0,1}, jj in 0..3: MFMA k index
// 8q + t is element 128c + 32q + 8jj + t of the step on both operands (weight
// word jj of chunk c; block scale 8c + 2q + jj/2), so the sums run over all
// of K.
#include "moe_ffn_common.hpp"
#include "moe_internal.hpp"
#include "moe_prefill_items.hpp"

namespace moe {

namespace {

constexpr int kFK = 256;           // K elements per step
constexpr int kFNW = 8;            // waves per block (two per SIMD)
constexpr int kFNB = 4;            // n-blocks of 16 weight rows per wave
constexpr int kFNH = kFNB / 2;     // gate (or up) n-blocks of a gate_up wave
constexpr int kFWR = 16 * kFNB * kFNW;  // weight rows per N tile (512)
constexpr int kFARow = 2 * kFK;    // bytes of one A row per step
constexpr int kFSRow = kFK / 16;   // scale bytes of one weight row per step
// Consecutive items per XCD (pf_item_of_block).  Measured, fused FFN at
// T=4096 / T=8192 (FP8 arm): 524 / 881 us with 1, 520 / 880 with 2, 515 /
// 846 with 4, 514 / 869 with 8.
constexpr int kFusedXcdRun = 4;

struct FfnSmem {
  uint8_t A[2][kPM * kFARow];        // A tile of a step (rows x 512 B), chunks swizzled by (row & 15)
  uint8_t S[2][kFWR * kFSRow];       // block scales of a step, tile row rho at 16 * rho
  unsigned long long base[kPMaxG];   // item table of pf_find_tile
  unsigned long long wsum[kFNW];
  float row_fac[kPM];  // gate_up epilogue factor of the row's token
  int row_ok[kPM];     // the row is a valid slot of the group
  uint32_t rowoff[kPM];  // byte offset of the row's A source (gate_up: token * 2H; down: r * 2I)
};

// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// no swizzle, no index stride): byte-addressed loads with range checking.
constexpr int kBufferFlags = 0x00020000;

// s_waitcnt limiting only the vector-memory counter to N (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14]; expcnt [6:4] and lgkmcnt [11:8] at max).
template <int N>
__device__ __forceinline__ void fused_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One projection of a work item: every N tile of it, K in steps of 256.
// GU = gate_up (A = f16 rows of xh by token, epilogue SiLU * up -> h),
// otherwise down (A = bf16 h rows of the tile, epilogue -> y).  NMB = valid
// 32-row blocks of the tile (2 * NMB m-blocks of 16).  ARES (down at K = 512):
// the two stages hold the whole h tile, loaded once in the prologue.
template <bool GU, int NMB, bool ARES>
__device__ __forceinline__ void fused_phase(FfnSmem& sm, const PfTile& ti,
                                            const uint8_t* __restrict__ codes_g,
                                            const uint8_t* __restrict__ scales_g,
                                            const float* __restrict__ scale2,
                                            const uint8_t* __restrict__ abase, uint32_t abytes,
                                            int H, int I, uint16_t* __restrict__ out) {
  constexpr int MB = 2 * NMB;
  constexpr int AI = NMB * 32 * kFARow / 1024 / kFNW;  // A DMA instructions per wave per step
  static_assert(!(GU && ARES), "the activation rows stream");
  // f16 MFMA (weights dequantised with one instruction per element) for
  // gate_up and for a resident h tile, which is turned into f16 in place;
  // bf16 MFMA for a streamed h tile
  constexpr bool F16 = GU || ARES;
  const int KD = GU ? H : I;
  const int nsteps = KD / kFK;
  const int NT = GU ? 2 * I / kFWR : H / kFWR;
  constexpr int NTROWS = GU ? kFWR / 2 : kFWR;  // weight rows one N tile advances (per half for gate_up)
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: LDS bases in SGPRs
  const int m16 = lane & 15, q = lane >> 4;
  const int e = ti.g;
  const uint32_t rowb = (uint32_t)KD / 2, srow = (uint32_t)KD / 16;

  // weight row (inside the group's matrix, N tile 0) of tile row
  // rho = 16 kFNB w + 16 nb + n: for gate_up, the wave's first kFNH n-blocks
  // are gate rows and the others the up rows of the same pairs
  auto row_of = [&](int rho) -> uint32_t {
    const int w = rho / (16 * kFNB), nb = (rho / 16) % kFNB, n = rho & 15;
    if (GU) return (uint32_t)((nb >= kFNH ? I : 0) + 16 * kFNH * w + 16 * (nb % kFNH) + n);
    return (uint32_t)rho;
  };
  // lane part of the weight offsets (n-block 0 of the wave); n-block nb adds
  // the uniform nb_off(nb)
  // (the per-lane offsets below are functions of the lane id, re-derived in
  // every step from an opaque copy of it instead of being held in registers
  // across the whole K loop)
  auto wlane_of = [&](int ln) -> uint32_t {
    return row_of(16 * kFNB * wv + (ln & 15)) * rowb + 16u * (uint32_t)(ln >> 4);
  };
  auto nb_off = [&](int nb) -> int {
    return (int)((row_of(16 * kFNB * wv + 16 * nb) - row_of(16 * kFNB * wv)) * rowb);
  };
  // scale DMA: instruction k (k = wv, wv + kFNW, ...) moves tile rows 64 k + lane
  constexpr int SI = kFWR * kFSRow / 1024 / kFNW;
  auto slane_of = [&](int ln) -> uint32_t { return row_of(64 * wv + ln) * srow; };
  auto s_off = [&](int i) -> int {  // uniform
    return (int)((row_of(64 * (wv + kFNW * i)) - row_of(64 * wv)) * srow);
  };
  // A DMA: instruction i of wave wv fills chunk positions 64 (wv + kFNW i) +
  // lane of the stage: row r = 2 (wv + kFNW i) + lane / 32, chunk position
  // lane % 32, which holds logical chunk (lane % 32) ^ (r & 15).  The source
  // offset is rowoff[r] + 16 chunk.
  auto ach = [&](int ln, int i) -> uint32_t {
    return 16u * (uint32_t)((ln & 31) ^ ((2 * (wv + kFNW * i) + (ln >> 5)) & 15));
  };

  // Buffer resources (every load is a 32-bit per-lane offset from a uniform
  // base, no 64-bit address registers; a read past the end returns zeros and
  // touches no memory).  `live` = false gives a resource of size 0: the loads
  // of a step that does not exist are issued without branching and fetch
  // nothing.
  const uint32_t wbytes = (GU ? 2 * I : H) * rowb, sbytes = (GU ? 2 * I : H) * srow;
  auto rsrc = [](const void* p, uint32_t bytes, bool live) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, live ? (int)bytes : 0, kBufferFlags);
  };

  // weight codes of chunk c (bytes [64c, 64c + 64) of each row's 128-byte
  // step slice) of all the wave's n-blocks, for N tile j, step s
  auto load_w = [&](u32x4 (&w)[kFNB], int c, int j, int s, bool live, int ln) {
    const uint32_t wlane = wlane_of(ln);
    const __amdgpu_buffer_rsrc_t rw = rsrc(codes_g, wbytes, live);
    const int so = j * NTROWS * (int)rowb + kFSRow * 8 * s;
#pragma unroll
    for (int nb = 0; nb < kFNB; ++nb)
      w[nb] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)wlane + 64 * c, so + nb_off(nb), 0);
  };
  auto dma_a = [&](int s, int st, bool live, int ln) {
    const uint32_t* rowoff_l = &sm.rowoff[2 * wv + (ln >> 5)];  // + 2 kFNW i for instruction i
    const __amdgpu_buffer_rsrc_t ra = rsrc(abase, abytes, live);
#pragma unroll
    for (int i = 0; i < AI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)&sm.A[st][1024 * (wv + kFNW * i)], 16,
          (int)(rowoff_l[2 * kFNW * i] + ach(ln, i)), kFARow * s, 0, 0);
  };
  auto dma_s = [&](int j, int s, int st, bool live, int ln) {
    const uint32_t slane = slane_of(ln);
    const __amdgpu_buffer_rsrc_t rs = rsrc(scales_g, sbytes, live);
    const int so = j * NTROWS * (int)srow + kFSRow * s;
#pragma unroll
    for (int i = 0; i < SI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)&sm.S[st][1024 * (wv + kFNW * i)], 16,
          (int)slane, so + s_off(i), 0, 0);
  };

  // A operand of m-block mb, sub-MFMA (c, jj): row 16 mb + m16, logical chunk
  // 16 c + 4 q + jj, stored at chunk (4 q + jj) ^ m16 of the row's half c
  auto aoff_of = [&](int ln, int jj) -> uint32_t {
    return (uint32_t)((ln & 15) * kFARow + 16 * ((4 * (ln >> 4) + jj) ^ (ln & 15)));
  };

  f32x4 acc[MB][kFNB];
  // Chunk c of the step (k-blocks 4c .. 4c + 3).  Per k-block, the A
  // operands of every m-block (each read feeds all kFNB n-blocks), then per
  // n-block its dequantised B operand and MFMAs.  The B operands rotate
  // through 3 register slots, so a dequant never overwrites an operand that a
  // queued MFMA has yet to read; the other wave on the SIMD covers the LDS
  // latency at the start of each k-block.
  auto compute = [&](const u32x4 (&w)[kFNB], int c, int st, int ln) {
    const uint8_t* Ab = sm.A[st] + 256 * c;
    const uint8_t* Sb = sm.S[st] + (16 * kFNB * wv + (ln & 15)) * kFSRow + 2 * (ln >> 4) + 8 * c;
    uint32_t sp[kFNB];
#pragma unroll
    for (int nb = 0; nb < kFNB; ++nb) sp[nb] = *(const uint16_t*)(Sb + 16 * kFSRow * nb);
    u32x4 bq[3];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x4 a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) a[mb] = *(const u32x4*)(Ab + aoff_of(ln, jj) + mb * 16 * kFARow);
#pragma unroll
      for (int nb = 0; nb < kFNB; ++nb) {
        u32x4& b = bq[(kFNB * jj + nb) % 3];
        if (F16) {
          const f16x2 sv = e4m3x2_to_f16(sp[nb]);
          b = __builtin_bit_cast(u32x4, dqh8(w[nb][jj], jj < 2 ? sv.x : sv.y));
        } else {
          const f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sp[nb], 1.0f, false);
          b = __builtin_bit_cast(u32x4, dq8(w[nb][jj], jj < 2 ? sv.x : sv.y));
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          // weights as the MFMA's A operand, tokens as B: the lane holding
          // token column t gets 4 consecutive output features of it
          if (F16)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8, b), __builtin_bit_cast(f16x8, a[mb]), acc[mb][nb], 0, 0, 0);
          else
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a[mb]), acc[mb][nb], 0, 0, 0);
        }
        if (nb % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
      // one k-block at a time: bounds the operands in flight
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One step from stage st, with no branch inside.  Step s + 1 (if any; else
  // the same loads against size-0 resources) is requested meanwhile: its A
  // tile and scales first (into the other stage), then the weights of chunk 0
  // once this step has consumed them, then those of chunk 1; the closing wait
  // leaves only those last kFNB weight loads in flight (their first use is
  // half-way through the next step).
  u32x4 w0[kFNB], w1[kFNB];
  const int total = NT * nsteps;
  auto step = [&](int j, int s, int st) {
    int ln = (int)(threadIdx.x & 63);
    asm volatile("" : "+v"(ln));
    const int gs = j * nsteps + s;
    const bool more = gs + 1 < total;
    const int jn = s + 1 < nsteps ? j : j + 1, sn = s + 1 < nsteps ? s + 1 : 0;
    if (!ARES) dma_a(sn, st ^ 1, more, ln);
    dma_s(jn, sn, st ^ 1, more, ln);
    compute(w0, 0, st, ln);
    load_w(w0, 0, jn, sn, more, ln);
    compute(w1, 1, st, ln);
    load_w(w1, 1, jn, sn, more, ln);
    fused_wait_vmcnt<kFNB>();
    __syncthreads();  // every wave's DMA has landed; stage st is free again
  };

  load_w(w0, 0, 0, 0, true, lane);
  load_w(w1, 1, 0, 0, true, lane);
  dma_a(0, 0, true, lane);
  if (ARES) dma_a(1, 1, true, lane);
  dma_s(0, 0, 0, true, lane);
  fused_wait_vmcnt<0>();
  __syncthreads();
  if (ARES) {
    // The resident bf16 h rows -> f16 in place, each row times the power of
    // two that brings its absmax into [2^14, 2^15) (exact for every value
    // above 2^-29 of the row's absmax), undone in the epilogue through
    // row_fac.  Row r's 512 elements are its 512-byte slices of the two
    // stages; lane l holds 16 bytes of stage l / 32 (the chunk swizzle does
    // not matter to an elementwise pass).
    for (int r = wv; r < MB * 16; r += kFNW) {
      uint8_t* p = &sm.A[lane >> 5][r * kFARow + 16 * (lane & 31)];
      const u32x4 v = *(const u32x4*)p;
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[k] & 0xFFFFu)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[k] >> 16)));
      }
      amax = wave_max_nonneg(amax);  // fmaxf drops NaN: every lane is >= 0, not NaN
      const int sh = f16_row_shift(amax);
      const float mul = ldexpf(1.0f, sh);
      if (lane == 0) sm.row_fac[r] = ldexpf(1.0f, -sh);
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = pack_f16x2(bf16_bits_to_f32(v[k] & 0xFFFFu) * mul, bf16_bits_to_f32(v[k] >> 16) * mul);
      *(u32x4*)p = o;
    }
    __syncthreads();
  }
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kFNB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // two steps per iteration (nsteps is even), so the stage of each is static
    for (int s = 0; s < nsteps; s += 2) {
      step(j, s, 0);
      step(j, s + 1, 1);
    }

    // ---- epilogue of N tile j ----
    // opaque copies (p0, and a zero added to the row-table indices): the
    // epilogue's addresses and row flags are rebuilt after each K loop instead
    // of being hoisted out of it into registers
    int p0 = ti.p0, z = 0;
    asm volatile("" : "+s"(p0), "+s"(z));
    // acc[mb][nb][v]: token row r = 16 mb + (lane % 16), output feature
    // 16 nb + 4 (lane / 16) + v of the wave's n-blocks: 4 consecutive
    // features per lane, stored as one 8-byte write
    const int ln = (int)(threadIdx.x & 63);
    const int r16 = ln & 15, g4 = 4 * (ln >> 4);
    if (GU) {
      const float s2g = scale2[3 * e + 0], s2u = scale2[3 * e + 1];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = 16 * mb + r16;
        if (r < ti.rows && sm.row_ok[r + z]) {
          const float f = sm.row_fac[r + z];
#pragma unroll
          for (int np = 0; np < kFNH; ++np) {
            const int col = NTROWS * j + 16 * kFNH * wv + 16 * np + g4;
            float hv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float g = acc[mb][np][v] * s2g * f, u = acc[mb][kFNH + np][v] * s2u * f;
              hv[v] = silu_f32(g) * u;
            }
            *(u32x2*)(out + (size_t)(p0 + r) * I + col) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
          }
        }
      }
    } else {
      const float s2d = scale2[3 * e + 2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = 16 * mb + r16;
        if (r < ti.rows && sm.row_ok[r + z]) {
          const float f = (ARES ? sm.row_fac[r + z] : 1.0f) * s2d;
#pragma unroll
          for (int nb = 0; nb < kFNB; ++nb) {
            const int col = NTROWS * j + 16 * kFNB * wv + 16 * nb + g4;
            const f32x4 v = acc[mb][nb];
            *(u32x2*)(out + (size_t)(p0 + r) * H + col) = u32x2{pack_bf16x2(v[0] * f, v[1] * f), pack_bf16x2(v[2] * f, v[3] * f)};
          }
        }
      }
    }
  }
}

template <int NMB>
__device__ __forceinline__ void fused_item(FfnSmem& sm, const PfTile& ti,
                                           const uint8_t* __restrict__ gu_codes,
                                           const uint8_t* __restrict__ gu_scales,
                                           const uint8_t* __restrict__ dn_codes,
                                           const uint8_t* __restrict__ dn_scales,
                                           const float* __restrict__ scale2,
                                           const _Float16* __restrict__ xh, uint32_t xbytes,
                                           int H, int I, uint16_t* __restrict__ h,
                                           uint16_t* __restrict__ y) {
  const size_t e = (size_t)ti.g;
  fused_phase<true, NMB, false>(sm, ti, gu_codes + e * 2 * I * (H / 2), gu_scales + e * 2 * I * (H / 16),
                         scale2, (const uint8_t*)xh, xbytes, H, I, h);
  // every wave's h stores are complete (vmcnt) and, after the barrier,
  // visible to the whole block; the down phase reads the tile's rows back
  fused_wait_vmcnt<0>();
  for (int r = threadIdx.x; r < kPM; r += 64 * kFNW) sm.rowoff[r] = r < ti.rows ? (uint32_t)r * I * 2 : 0u;
  __syncthreads();
  const uint8_t* dc = dn_codes + e * H * (I / 2);
  const uint8_t* dsc = dn_scales + e * H * (I / 16);
  const uint8_t* hb = (const uint8_t*)(h + (size_t)ti.p0 * I);
  const uint32_t hbytes = (uint32_t)ti.rows * I * 2;
  if (I == 2 * kFK)
    fused_phase<false, NMB, true>(sm, ti, dc, dsc, scale2, hb, hbytes, H, I, y);
  else
    fused_phase<false, NMB, false>(sm, ti, dc, dsc, scale2, hb, hbytes, H, I, y);
}

__global__ __launch_bounds__(64 * kFNW, 1) void k_prefill_ffn(
    const uint8_t* __restrict__ gu_codes, const uint8_t* __restrict__ gu_scales,
    const uint8_t* __restrict__ dn_codes, const uint8_t* __restrict__ dn_scales,
    const float* __restrict__ scale2, const _Float16* __restrict__ xh,
    const float* __restrict__ rowfac, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slot, int T, int K, int H, int I, int G, int has_shared,
    int shared_rows, uint16_t* __restrict__ h, uint16_t* __restrict__ y) {
  constexpr int NTHR = 64 * kFNW;
  __shared__ __align__(16) FfnSmem sm;
  // activation rows [T + shared_rows][H]: the shared group reads rows
  // shared_rows + t (its own activation arm) when shared_rows > 0
  const uint32_t xbytes = (uint32_t)(T + shared_rows) * (uint32_t)H * 2u;  // < 2^31 (fused_supported)
  PfTile ti;
  if (!pf_find_tile<NTHR>(offsets, G, 1, sm.base, sm.wsum, &ti, kFusedXcdRun)) return;
  const int roff = (has_shared && ti.g == G - 1) ? shared_rows : 0;
  for (int r = threadIdx.x; r < kPM; r += NTHR) {
    int tk = -1;
    if (r < ti.rows) tk = slot_token(sorted_slot[ti.p0 + r], T, K, has_shared);
    sm.row_ok[r] = tk >= 0;
    sm.rowoff[r] = tk >= 0 ? (uint32_t)(tk + roff) * (uint32_t)H * 2u : 0u;  // row 0 for padding rows
    sm.row_fac[r] = tk >= 0 ? rowfac[tk + roff] : 0.f;
  }
  __syncthreads();
  switch ((ti.rows + 31) / 32) {  // uniform per block
    case 1: fused_item<1>(sm, ti, gu_codes, gu_scales, dn_codes, dn_scales, scale2, xh, xbytes, H, I, h, y); break;
    case 2: fused_item<2>(sm, ti, gu_codes, gu_scales, dn_codes, dn_scales, scale2, xh, xbytes, H, I, h, y); break;
    case 3: fused_item<3>(sm, ti, gu_codes, gu_scales, dn_codes, dn_scales, scale2, xh, xbytes, H, I, h, y); break;
    default: fused_item<4>(sm, ti, gu_codes, gu_scales, dn_codes, dn_scales, scale2, xh, xbytes, H, I, h, y); break;
  }
}

}  // namespace

void register_fused_kernels(std::vector<const void*>& k) { k.push_back((const void*)&k_prefill_ffn); }

// The fused kernel's shape rules: N tiles of 512 weight rows (2I and H), an
// even number of K steps of 256 (H and I), and 32-bit byte offsets inside the activation rows
// (T * H * 2) and the h rows of one tile.
bool fused_supported(int T, int H, int I) {
  return H % 512 == 0 && I % 512 == 0 && (long long)T * H * 2 < (1LL << 31);
}

hipError_t launch_prefill_fused(const moe_nvfp4_weights& W, int T, int K, const int32_t* offsets,
                                const int32_t* sorted_slot, const _Float16* xh,
                                const float* rowfac, int shared_rows, uint16_t* hbuf, uint16_t* y,
                                hipStream_t s) {
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const int G = W.E + hs;
  const long S = (long)T * K + (hs ? T : 0);
  const long items = S / kPM + G;  // at most S/128 full row tiles plus one partial tile per group
  MOE_LAUNCH("grouped_ffn", s, k_prefill_ffn, dim3((unsigned)items), dim3(64 * kFNW), 0, s,
             W.gu_codes, W.gu_scales, W.dn_codes, W.dn_scales, W.scale2, xh, rowfac, offsets,
             sorted_slot, T, K, H, I, G, hs, shared_rows, hbuf, y);
  return hipGetLastError();
}

}  // namespace moe
