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

hipError_t launch_expert_ffn(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                             const int32_t* offsets, const int32_t* sorted_slot,
                             const int32_t* groups, int act_mode, uint16_t* y, void* ws,
                             hipStream_t s) {
  const int H = W.H, I = W.I, hs = W.has_shared ? 1 : 0;
  const size_t S = (size_t)T * K + (hs ? (size_t)T : 0);
  uint8_t* wp = (uint8_t*)ws;
  uint16_t* hbuf = (uint16_t*)wp;
  wp += align256(S * I * sizeof(uint16_t));
  uint8_t* xq = nullptr;
  float* xs = nullptr;
  if (act_mode != MOE_ACT_BF16) {
    xq = wp;
    wp += align256((size_t)T * H);
    xs = (float*)wp;
    wp += align256((size_t)T * sizeof(float));
  }
  if (T <= kDecodeMaxT && decode_supported(H, I))
    return launch_decode_ffn(W, x, T, K, offsets, sorted_slot, groups, act_mode, hbuf, xq, xs, y, s);
  const bool mixed = mixed_arm(act_mode);
  const int rows = mixed ? 2 * T : T;
  _Float16* xh = (_Float16*)wp;
  float* rowfac = (float*)(wp + align256((size_t)rows * H * sizeof(_Float16)));
  hipError_t e;
  if (!mixed) {
    e = launch_xprep(x, T, H, act_mode == MOE_ACT_FP8_ROW, xh, rowfac, xq, xs, s);
  } else {  // rows [0, T): the routed experts' form; rows [T, 2T): the shared expert's
    e = launch_xprep(x, T, H, act_mode == MOE_ACT_FP8_ROUTED, xh, rowfac, xq, xs, s);
    if (e == hipSuccess)
      e = launch_xprep(x, T, H, act_mode == MOE_ACT_FP8_SHARED, xh + (size_t)T * H, rowfac + T,
                       xq, xs, s);
  }
  if (e != hipSuccess) return e;
  const int shared_rows = mixed ? T : 0;
  if (fused_supported(rows, H, I))
    return launch_prefill_fused(W, T, K, offsets, sorted_slot, xh, rowfac, shared_rows, hbuf, y, s);
  return launch_prefill_ffn(W, T, K, offsets, sorted_slot, xh, rowfac, shared_rows, hbuf, y, s);
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
// run three kernels (routing + permutation + gate_up, down, combine); other
// calls run route+permute, then the expert FFN and the combine.  The
// workspace serves the permutation first and the FFN after it (stream order).
size_t layer_workspace_bytes(int T, int E, int K, int H, int I, int has_shared, int act_mode) {
  const size_t a = permute_workspace_bytes(T, E, K);
  const size_t b = ffn_combine_workspace_bytes(T, K, H, I, has_shared, act_mode);
  return a > b ? a : b;
}

hipError_t launch_layer(const moe_nvfp4_weights& W, const float* logits, const uint16_t* x, int T,
                        int K, int act_mode, const float* gate, const RpOut& ro,
                        uint16_t* y_slots, uint16_t* out, void* ws, hipStream_t s) {
  const int H = W.H, I = W.I, E = W.E, hs = W.has_shared ? 1 : 0;
  if (decode_layer_supported(T, E, K, H, I, act_mode)) {
    const size_t S = (size_t)T * K + (hs ? (size_t)T : 0);
    uint8_t* wp = (uint8_t*)ws;
    uint16_t* hbuf = (uint16_t*)wp;
    wp += align256(S * I * sizeof(uint16_t));
    uint8_t* xq = nullptr;
    float* xs = nullptr;
    if (act_mode != MOE_ACT_BF16) {
      xq = wp;
      wp += align256((size_t)T * H);
      xs = (float*)wp;
    }
    return launch_decode_layer(W, logits, x, T, K, act_mode, gate, ro, hbuf, xq, xs, y_slots, out,
                               s);
  }
  hipError_t e = launch_route_permute(logits, T, E, K, hs, ro.ids, ro.w, ro.counts, ro.offsets,
                                      ro.sorted_slot, ro.slot_pos, ro.groups, ws, s);
  if (e != hipSuccess) return e;
  return launch_expert_ffn_combine(W, x, T, K, ro.offsets, ro.sorted_slot, ro.groups, act_mode,
                                   ro.w, ro.slot_pos, gate, y_slots, out, ws, s);
}

}  // namespace moe
