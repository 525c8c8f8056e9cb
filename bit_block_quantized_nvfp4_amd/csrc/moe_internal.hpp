// Host-side declarations shared by the library's translation units: kernel
// launchers (one per kernel family), the kernel registry used by moe_init(),
// and the launch bracket used for per-kernel timing.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/moe_nvfp4.h"

namespace moe {

// Per-kernel timing (see moe_timing_* in the public header). timing_begin
// returns a record slot (or -1 when timing is off) that timing_end closes.
int timing_begin(const char* name, hipStream_t s);
void timing_end(int slot, hipStream_t s);

#define MOE_LAUNCH(name, stream, ...)                 \
  do {                                                \
    int moe_slot_ = ::moe::timing_begin(name, stream); \
    hipLaunchKernelGGL(__VA_ARGS__);                  \
    ::moe::timing_end(moe_slot_, stream);             \
  } while (0)

// Kernel registries: every translation unit lists its __global__ functions so
// that moe_init() can resolve each of them once.
void register_route_kernels(std::vector<const void*>& k);
void register_permute_kernels(std::vector<const void*>& k);
void register_combine_kernels(std::vector<const void*>& k);
void register_ffn_kernels(std::vector<const void*>& k);

// Launchers. Arguments are validated by the C entry points before these run.
hipError_t launch_route_topk(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                             hipStream_t s);
// One activation arm of the grouped path's prep: f16 rows and epilogue
// factors, e4m3 row quantisation when fp8 != 0.
struct XprepArm {
  _Float16* xh;
  float* unmul;
  int fp8;
};
// launch_route_topk and launch_xprep of one or two arms (b.xh == nullptr: one)
// as one launch (moe_route.hip).
hipError_t launch_route_xprep(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                              const uint16_t* x, int H, XprepArm a, XprepArm b, uint8_t* xq,
                              float* xs, hipStream_t s);

size_t permute_workspace_bytes(int T, int E, int K);
// Batches up to this many tokens (one per wave) are routed and permuted by
// one block.
constexpr int kRouteFuseMaxT = 8;
hipError_t launch_route_permute(const float* logits, int T, int E, int K, int has_shared,
                                int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                                int32_t* sorted_slot, int32_t* slot_pos, int32_t* groups, void* ws,
                                hipStream_t s);
hipError_t launch_permute(const int32_t* ids, int T, int E, int K, int has_shared,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                          int32_t* slot_pos, int32_t* groups, void* ws, hipStream_t s);

hipError_t launch_combine(const uint16_t* y, const float* w, const int32_t* slot_pos,
                          const float* gate, int T, int K, int H, int has_shared, uint16_t* out,
                          hipStream_t s);

void register_router_kernels(std::vector<const void*>& k);
hipError_t launch_router_topk(const moe_nvfp4_router& R, const uint16_t* x, int T, int K,
                              int32_t* ids, float* w, float* logits, float* gate, hipStream_t s);

size_t ffn_workspace_bytes(int T, int K, int H, int I, int has_shared, int act_mode);
hipError_t launch_expert_ffn(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                             const int32_t* offsets, const int32_t* sorted_slot,
                             const int32_t* groups, int act_mode, uint16_t* y_slots, void* ws,
                             hipStream_t s);

size_t ffn_combine_workspace_bytes(int T, int K, int H, int I, int has_shared, int act_mode);
hipError_t launch_expert_ffn_combine(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                                     const int32_t* offsets, const int32_t* sorted_slot,
                                     const int32_t* groups, int act_mode, const float* w,
                                     const int32_t* slot_pos, const float* gate,
                                     uint16_t* y_slots, uint16_t* out, void* ws, hipStream_t s);

// Decode/prefill switch of moe_expert_ffn: T <= kDecodeMaxT uses the GEMV path.
constexpr int kDecodeMaxT = 8;

// Compute units of the current device (cached per device by the API layer).
int num_cus();

void register_decode_kernels(std::vector<const void*>& k);
void register_prefill_kernels(std::vector<const void*>& k);
// Per-row activation prep shared by both regimes: f16 rows xh [T][H] (bf16
// arm: x * 2^sh with unmul = 2^-sh; FP8 arm: the exact f16 value of each e4m3
// code with unmul = the row scale, codes and scales also written to xq, xs).
hipError_t launch_xprep(const uint16_t* x, int T, int H, bool fp8, _Float16* xh, float* unmul,
                        uint8_t* xq, float* xs, hipStream_t s);
hipError_t launch_prefill_ffn(const moe_nvfp4_weights& W, int T, int K, const int32_t* offsets,
                              const int32_t* sorted_slot, const _Float16* xh, const float* rowfac,
                              int shared_rows, uint16_t* hbuf, uint16_t* y, hipStream_t s);
// Fused gate_up -> SiLU -> down in one launch (moe_ffn_fused.hip) for the
// shapes fused_supported() accepts; the two-launch grouped GEMM otherwise.
void register_fused_kernels(std::vector<const void*>& k);
bool fused_supported(int T, int H, int I);
hipError_t launch_prefill_fused(const moe_nvfp4_weights& W, int T, int K, const int32_t* offsets,
                                const int32_t* sorted_slot, const _Float16* xh,
                                const float* rowfac, int shared_rows, uint16_t* hbuf, uint16_t* y,
                                hipStream_t s);
bool decode_supported(int H, int I);
size_t xprep_workspace_bytes(int T, int H);
// The permutation's global outputs (the layout of moe_route_permute).
struct RpOut {
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slot;
  int32_t* slot_pos;
  int32_t* groups;
};
// The decode layer kernels (routing and permutation inside the gate_up
// launch, then down and combine): batches of up to kRouteFuseMaxT tokens, the
// bf16 and the FP8 row arms, decode-supported H and I.
bool decode_layer_supported(int T, int E, int K, int H, int I, int act_mode);
hipError_t launch_decode_layer(const moe_nvfp4_weights& W, const float* logits, const uint16_t* x,
                               int T, int K, int act_mode, const float* gate, const RpOut& ro,
                               uint16_t* hbuf, uint8_t* xq, float* xs, uint16_t* y,
                               uint16_t* out, hipStream_t s);
// The whole layer (moe_layer): the decode layer kernels and the combine, or
// route+permute and the expert FFN + combine.
size_t layer_workspace_bytes(int T, int E, int K, int H, int I, int has_shared, int act_mode);
hipError_t launch_layer(const moe_nvfp4_weights& W, const float* logits, const uint16_t* x, int T,
                        int K, int act_mode, const float* gate, const RpOut& ro,
                        uint16_t* y_slots, uint16_t* out, void* ws, hipStream_t s);
hipError_t launch_decode_ffn(const moe_nvfp4_weights& W, const uint16_t* x, int T, int K,
                             const int32_t* offsets, const int32_t* sorted_slot,
                             const int32_t* groups, int act_mode, uint16_t* hbuf, uint8_t* xq,
                             float* xs, uint16_t* y, hipStream_t s);

}  // namespace moe
