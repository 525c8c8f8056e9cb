// Expert FFN of the NVFP4 MoE layer (A3-A9): workspace layout and the
// dispatch between the decode multi-row GEMV (T <= 8, moe_ffn_decode.hip) and
// the prefill grouped GEMM (moe_ffn_prefill.hip).
//
// Numerics (the table attributing the transposed-MoE perplexity gap in the
// issue "[job] Qwen3.8-Flash-Next: long-context cold prefill to SGLang
// parity"): weights are dequantised as e2m1 x e4m3 block scale, exactly (at
// most 6 significant bits, exponents 2^-10 .. 2^12, so exact in f16 and bf16),
// the products run on MFMA with f32 accumulation, scale2 (and the FP8 row
// scale) multiply the f32 sums, SiLU(gate) * up is stored as bf16, the down
// output is stored as bf16 per sorted slot.
//
// Both regimes first turn each activation row into f16 (k_dec_xprep): the
// bf16 arm multiplies the row by a power of two that brings its absmax into
// [2^14, 2^15) (exact for every value above 2^-29 of the row's absmax; the
// shift is undone in the f32 epilogue), the FP8 arm quantises the row to e4m3
// (s_t = absmax / 448) and keeps the exact f16 value of each code with s_t as
// the epilogue factor.  gate_up then runs on f16 MFMA against weights
// dequantised to f16 with one instruction per element; down runs on bf16 MFMA
// against the bf16 h rows.
#include <math.h>

#include "moe_ffn_common.hpp"
#include "moe_internal.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
void register_ffn_kernels(std::vector<const void*>& k) {
  register_prefill_kernels(k);
  register_fused_kernels(k);
  register_decode_kernels(k);
}

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Per-class arms: the routed and the shared expert read different activation
// forms, kept as one [2T][H] array (rows T.. for the shared group).
static inline bool mixed_arm(int act_mode) {
  return act_mode == MOE_ACT_FP8_ROUTED || act_mode == MOE_ACT_FP8_SHARED;
}

size_t ffn_workspace_bytes(int T, int K, int H, int I, int has_shared, int act_mode) {
  const size_t S = (size_t)T * K + (has_shared ? (size_t)T : 0);
  size_t b = align256(S * I * sizeof(uint16_t));
  if (act_mode != MOE_ACT_BF16) b += align256((size_t)T * H) + align256((size_t)T * sizeof(float));
  return b + xprep_workspace_bytes(mixed_arm(act_mode) ? 2 * T : T, H);
}

namespace {

// The expert FFN's workspace: the h rows [S][I] bf16 first, then for the FP8
// arms the e4m3 rows [T][H] and row scales [T], then for the grouped path the
// f16 rows and their epilogue factors ([T][H] and [T], or [2T][H] and [2T]
// for the mixed arms: rows T.. for the shared expert).
struct FfnWs {
  uint16_t* hbuf;
  uint8_t* xq;
  float* xs;
  _Float16* xh;
  float* rowfac;
  size_t prep_off;  // byte offset of everything after the h rows
};

FfnWs ffn_ws(void* ws, int T, int K, int H, int I, int has_shared, int act_mode) {
  const size_t S = (size_t)T * K + (has_shared ? (size_t)T : 0);
  uint8_t* wp = (uint8_t*)ws;
  FfnWs b{};
  b.hbuf = (uint16_t*)wp;
  b.prep_off = align256(S * I * sizeof(uint16_t));
  wp += b.prep_off;
  if (act_mode != MOE_ACT_BF16) {
    b.xq = wp;
    wp += align256((size_t)T * H);
    b.xs = (float*)wp;
    wp += align256((size_t)T * sizeof(float));
  }
  const int rows = mixed_arm(act_mode) ? 2 * T : T;
  b.xh = (_Float16*)wp;
  b.rowfac = (float*)(wp + align256((size_t)rows * H * sizeof(_Float16)));
  return b;
}

// The grouped path's activation arms: one, or for the mixed arms the routed
// experts' form (rows [0, T)) and the shared expert's (rows [T, 2T)).
void xprep_arms(const FfnWs& b, int T, int H, int act_mode, XprepArm& a, XprepArm& a2) {
  if (!mixed_arm(act_mode)) {
    a = XprepArm{b.xh, b.rowfac, act_mode == MOE_ACT_FP8_ROW ? 1 : 0};
    a2 = XprepArm{nullptr, nullptr, 0};
  } else {
    a = XprepArm{b.xh, b.rowfac, act_mode == MOE_ACT_FP8_ROUTED ? 1 : 0};
    a2 = XprepArm{b.xh + (size_t)T * H, b.rowfac + T, act_mode == MOE_ACT_FP8_SHARED ? 1 : 0};
  }
}

bool ffn_is_grouped(int T, int H, int I) { return !(T <= kDecodeMaxT && decode_supported(H, I)); }

// The grouped path after its activation prep.
hipError_t launch_grouped_ffn(const moe_nvfp4_weights& W, int T, int K, const int32_t* offsets,
                              const int32_t* sorted_slot, int act_mode, const FfnWs& b,
                              uint16_t* y, hipStream_t s) {
  const int H = W.H, I = W.I;
  const bool mixed = mixed_arm(act_mode);
  const int shared_rows = mixed ? T : 0;
  if (fused_supported(mixed ? 2 * T : T, H, I))
    return launch_prefill_fused(W, T, K, offsets, sorted_slot, b.xh, b.rowfac, shared_rows,
                                b.hbuf, y, s);
  return launch_prefill_ffn(W, T, K, offsets, sorted_slot, b.xh, b.rowfac, shared_rows, b.hbuf,
                            y, s);
}

}  // namespace

hipError_t launch_expert_ffn(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                             const int32_t* offsets, const int32_t* sorted_slot,
                             const int32_t* groups, int act_mode, uint16_t* y, void* ws,
                             hipStream_t s) {
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const FfnWs b = ffn_ws(ws, T, K, H, I, hs, act_mode);
  if (!ffn_is_grouped(T, H, I))
    return launch_decode_ffn(W, x, T, K, offsets, sorted_slot, groups, act_mode, b.hbuf, b.xq,
                             b.xs, y, s);
  XprepArm a, a2;
  xprep_arms(b, T, H, act_mode, a, a2);
  hipError_t e = launch_xprep(x, T, H, a.fp8 != 0, a.xh, a.unmul, b.xq, b.xs, s);
  if (e == hipSuccess && a2.xh) e = launch_xprep(x, T, H, a2.fp8 != 0, a2.xh, a2.unmul, b.xq, b.xs, s);
  if (e != hipSuccess) return e;
  return launch_grouped_ffn(W, T, K, offsets, sorted_slot, act_mode, b, y, s);
}

// The expert FFN followed by the combine kernel, as one call.  (Folding the
// combine into the decode down kernel -- the last block of each column slice
// combining it after the others publish their rows -- was measured slower:
// publishing across the XCDs' L2 caches costs a write-back per block, more
// than the combine launch it saves.)
size_t ffn_combine_workspace_bytes(int T, int K, int H, int I, int has_shared, int act_mode) {
  return ffn_workspace_bytes(T, K, H, I, has_shared, act_mode);
}

hipError_t launch_expert_ffn_combine(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                                     const int32_t* offsets, const int32_t* sorted_slot,
                                     const int32_t* groups, int act_mode, const float* w,
                                     const int32_t* slot_pos, const float* gate,
                                     uint16_t* y_slots, uint16_t* out, void* ws, hipStream_t s) {
  hipError_t e = launch_expert_ffn(W, x, T, K, offsets, sorted_slot, groups, act_mode, y_slots, ws, s);
  if (e != hipSuccess) return e;
  return launch_combine(y_slots, w, slot_pos, gate, T, K, W.H, W.has_shared ? 1 : 0, out, s);
}

// The whole layer in one call.  Decode batches of the bf16 or FP8 row arm
// run three kernels (routing + permutation + gate_up, down, combine).  Larger
// batches on the grouped path run the routing and the activation prep as one
// launch, then the permutation, the grouped FFN and the combine.  Other calls
// run route+permute, then the expert FFN and the combine.  The workspace
// serves the permutation first and the FFN after it (stream order); the
// activation prep's part of it lies after the permutation's.
size_t layer_workspace_bytes(int T, int E, int K, int H, int I, int has_shared, int act_mode) {
  const size_t a = permute_workspace_bytes(T, E, K);
  const size_t b = ffn_combine_workspace_bytes(T, K, H, I, has_shared, act_mode);
  return a > b ? a : b;
}

hipError_t launch_layer(const moe_nvfp4_weights& W, const float* logits, const uint16_t* x, int T,
                        int K, int act_mode, const float* gate, const RpOut& ro,
                        uint16_t* y_slots, uint16_t* out, void* ws, hipStream_t s) {
  const int H = W.H, I = W.I, E = W.E, hs = W.has_shared ? 1 : 0;
  const FfnWs b = ffn_ws(ws, T, K, H, I, hs, act_mode);
  if (decode_layer_supported(T, E, K, H, I, act_mode))
    return launch_decode_layer(W, logits, x, T, K, act_mode, gate, ro, b.hbuf, b.xq, b.xs, y_slots,
                               out, s);
  if (T > kRouteFuseMaxT && ffn_is_grouped(T, H, I) && permute_workspace_bytes(T, E, K) <= b.prep_off) {
    // the routing and the activation prep in one launch (their outputs lie
    // after the permutation's part of the workspace), then the permutation,
    // the grouped FFN and the combine
    XprepArm a, a2;
    xprep_arms(b, T, H, act_mode, a, a2);
    hipError_t e = launch_route_xprep(logits, T, E, K, ro.ids, ro.w, x, H, a, a2, b.xq, b.xs, s);
    if (e == hipSuccess)
      e = launch_permute(ro.ids, T, E, K, hs, ro.counts, ro.offsets, ro.sorted_slot, ro.slot_pos,
                         ro.groups, ws, s);
    if (e == hipSuccess)
      e = launch_grouped_ffn(W, T, K, ro.offsets, ro.sorted_slot, act_mode, b, y_slots, s);
    if (e != hipSuccess) return e;
    return launch_combine(y_slots, ro.w, ro.slot_pos, gate, T, K, H, hs, out, s);
  }
  hipError_t e = launch_route_permute(logits, T, E, K, hs, ro.ids, ro.w, ro.counts, ro.offsets,
                                      ro.sorted_slot, ro.slot_pos, ro.groups, ws, s);
  if (e != hipSuccess) return e;
  return launch_expert_ffn_combine(W, x, T, K, ro.offsets, ro.sorted_slot, ro.groups, act_mode,
                                   ro.w, ro.slot_pos, gate, y_slots, out, ws, s);
}

}  // namespace moe
