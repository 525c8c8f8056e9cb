// C entry points of libmoe_nvfp4: argument checks, the gfx950 gate, one-time
// kernel resolution, dispatch to the launchers, error text, and the optional
// per-kernel event timing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "moe_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MOE_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
std::mutex g_init_mu;
int g_init_state[kMaxDevices];  // 0 = not yet, 1 = ready, < 0 = status of the failure
std::string g_init_msg[kMaxDevices];
int g_cus[kMaxDevices];

// Workspace of moe_expert_ffn_noalloc: one copy per device, held until the
// process ends.  In host code `scratch` is only a stand-in for the symbol; its
// device address on each GPU is g_scratch[dev], taken once at init.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_WS_BYTES];
void* g_scratch[kMaxDevices];

int ensure_init() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_init_mu);
  if (g_init_state[dev] == 1) return MOE_OK;
  if (g_init_state[dev] < 0) {
    g_err = g_init_msg[dev];
    return g_init_state[dev];
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    int rc = fail(MOE_EUNSUPPORTED,
                  "moe_nvfp4 is built for gfx950 (MI355X) only; device %d is %s", dev,
                  prop.gcnArchName);
    g_init_state[dev] = rc;
    g_init_msg[dev] = g_err;
    return rc;
  }
  g_cus[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      int rc = e != hipSuccess ? hip_fail(e, "hipGetSymbolAddress(scratch) at init")
                               : fail(MOE_EHIP, "hipGetSymbolAddress(scratch) returned null");
      g_init_state[dev] = rc;
      g_init_msg[dev] = g_err;
      return rc;
    }
    g_scratch[dev] = p;
  }
  std::vector<const void*> ks;
  moe::register_route_kernels(ks);
  moe::register_router_kernels(ks);
  moe::register_permute_kernels(ks);
  moe::register_combine_kernels(ks);
  moe::register_ffn_kernels(ks);
  for (const void* k : ks) {
    hipFuncAttributes attr;
    e = hipFuncGetAttributes(&attr, k);
    if (e != hipSuccess) {
      int rc = hip_fail(e, "kernel lookup at init");
      g_init_state[dev] = rc;
      g_init_msg[dev] = g_err;
      return rc;
    }
  }
  g_init_state[dev] = 1;
  return MOE_OK;
}

// ---- timing ----
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
};
std::atomic<bool> g_timing_on{false};
std::mutex g_tmu;
std::vector<TimingRec> g_pool;
size_t g_used = 0;
long g_dropped = 0;
constexpr size_t kMaxRecords = 65536;

bool sizes_ok_common(int T, int E, int K) {
  return T >= 1 && E >= 1 && E <= 1024 && K >= 1 && K <= 32 && K <= E &&
         (long long)T * K <= (1LL << 30) && (long long)T * E <= (1LL << 40);
}

}  // namespace

namespace moe {

int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices || g_cus[dev] <= 0) return 256;
  return g_cus[dev];
}

int timing_begin(const char* name, hipStream_t s) {
  if (!g_timing_on.load(std::memory_order_relaxed)) return -1;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_used >= kMaxRecords) {
    ++g_dropped;
    return -1;
  }
  if (g_used == g_pool.size()) {
    TimingRec r{name, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess) return -1;
    if (hipEventCreate(&r.b) != hipSuccess) {
      (void)hipEventDestroy(r.a);
      return -1;
    }
    g_pool.push_back(r);
  }
  TimingRec& r = g_pool[g_used];
  r.name = name;
  if (hipEventRecord(r.a, s) != hipSuccess) return -1;
  return (int)g_used++;
}

void timing_end(int slot, hipStream_t s) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  (void)hipEventRecord(g_pool[(size_t)slot].b, s);
}

}  // namespace moe

extern "C" {

int moe_init(void) {
  const int rc = ensure_init();
  return rc == MOE_OK ? ok() : rc;
}

const char* moe_last_error(void) { return g_err.c_str(); }

size_t moe_workspace_bytes(int op, int T, int E, int K, int H, int I, int has_shared,
                           int act_mode) {
  if (!sizes_ok_common(T, E, K) || (has_shared != 0 && has_shared != 1)) return 0;
  if (op == MOE_OP_PERMUTE) return moe::permute_workspace_bytes(T, E, K);
  if (op == MOE_OP_LAYER) {
    if (H <= 0 || I <= 0 || act_mode < MOE_ACT_BF16 || act_mode > MOE_ACT_FP8_SHARED) return 0;
    return moe::layer_workspace_bytes(T, E, K, H, I, has_shared, act_mode);
  }
  if (op == MOE_OP_EXPERT_FFN || op == MOE_OP_EXPERT_FFN_COMBINE) {
    if (H <= 0 || I <= 0 || act_mode < MOE_ACT_BF16 || act_mode > MOE_ACT_FP8_SHARED) return 0;
    return op == MOE_OP_EXPERT_FFN ? moe::ffn_workspace_bytes(T, K, H, I, has_shared, act_mode)
                                   : moe::ffn_combine_workspace_bytes(T, K, H, I, has_shared, act_mode);
  }
  return 0;
}

int moe_route_topk(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                   void* stream) {
  if (!logits || !ids || !w) return fail(MOE_EINVAL, "moe_route_topk: null pointer");
  if (!sizes_ok_common(T, E, K))
    return fail(MOE_EINVAL, "moe_route_topk: need T >= 1, 1 <= K <= min(E, 32), E <= 1024 (T=%d E=%d K=%d)", T, E, K);
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  hipError_t e = moe::launch_route_topk(logits, T, E, K, ids, w, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_route_topk launch");
}

int moe_permute(const int32_t* ids, int T, int E, int K, int has_shared, int32_t* counts,
                int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, int32_t* groups,
                void* ws, size_t ws_bytes, void* stream) {
  if (!ids || !counts || !offsets || !sorted_slot || !slot_pos || !groups)
    return fail(MOE_EINVAL, "moe_permute: null pointer");
  if (!sizes_ok_common(T, E, K) || (has_shared != 0 && has_shared != 1))
    return fail(MOE_EINVAL, "moe_permute: need T >= 1, 1 <= K <= min(E, 32), E <= 1024, has_shared in {0,1}");
  const size_t need = moe::permute_workspace_bytes(T, E, K);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_EWORKSPACE, "moe_permute: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  hipError_t e = moe::launch_permute(ids, T, E, K, has_shared, counts, offsets, sorted_slot,
                                     slot_pos, groups, ws, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_permute launch");
}

int moe_expert_ffn(const moe_nvfp4_weights* W, const uint16_t* x, int T, int K,
                   const int32_t* offsets, const int32_t* sorted_slot, const int32_t* groups,
                   int act_mode, uint16_t* y_slots, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !x || !offsets || !sorted_slot || !groups || !y_slots)
    return fail(MOE_EINVAL, "moe_expert_ffn: null pointer");
  if (!W->gu_codes || !W->gu_scales || !W->dn_codes || !W->dn_scales || !W->scale2)
    return fail(MOE_EINVAL, "moe_expert_ffn: null weight pointer");
  if (act_mode < MOE_ACT_BF16 || act_mode > MOE_ACT_FP8_SHARED)
    return fail(MOE_EUNSUPPORTED, "moe_expert_ffn: unknown act_mode %d", act_mode);
  if (!sizes_ok_common(T, W->E, K) || (W->has_shared != 0 && W->has_shared != 1))
    return fail(MOE_EINVAL, "moe_expert_ffn: need T >= 1, 1 <= K <= min(E, 32), E <= 1024, has_shared in {0,1}");
  if (W->H < 256 || W->H > 4096 || W->H % 256 != 0 || W->I < 128 || W->I > 1024 || W->I % 128 != 0)
    return fail(MOE_EINVAL, "moe_expert_ffn: need H a multiple of 256 in [256, 4096] and I a multiple of 128 in [128, 1024] (H=%d I=%d)", W->H, W->I);
  const size_t need = moe::ffn_workspace_bytes(T, K, W->H, W->I, W->has_shared, act_mode);
  if (!ws || ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_expert_ffn: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  hipError_t e = moe::launch_expert_ffn(*W, x, T, K, offsets, sorted_slot, groups, act_mode,
                                        y_slots, ws, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_expert_ffn launch");
}

int moe_expert_ffn_noalloc(const moe_nvfp4_weights* W, const uint16_t* x, int T, int K,
                           const int32_t* offsets, const int32_t* sorted_slot,
                           const int32_t* groups, int act_mode, uint16_t* y_slots,
                           void* stream) {
  if (!W || !x || !offsets || !sorted_slot || !groups || !y_slots)
    return fail(MOE_EINVAL, "moe_expert_ffn_noalloc: null pointer");
  if (!W->gu_codes || !W->gu_scales || !W->dn_codes || !W->dn_scales || !W->scale2)
    return fail(MOE_EINVAL, "moe_expert_ffn_noalloc: null weight pointer");
  if (act_mode < MOE_ACT_BF16 || act_mode > MOE_ACT_FP8_SHARED)
    return fail(MOE_EUNSUPPORTED, "moe_expert_ffn_noalloc: unknown act_mode %d", act_mode);
  if (!sizes_ok_common(T, W->E, K) || (W->has_shared != 0 && W->has_shared != 1))
    return fail(MOE_EINVAL, "moe_expert_ffn_noalloc: need T >= 1, 1 <= K <= min(E, 32), E <= 1024, has_shared in {0,1}");
  if (W->H < 256 || W->H > 4096 || W->H % 256 != 0 || W->I < 128 || W->I > 1024 || W->I % 128 != 0)
    return fail(MOE_EINVAL, "moe_expert_ffn_noalloc: need H a multiple of 256 in [256, 4096] and I a multiple of 128 in [128, 1024] (H=%d I=%d)", W->H, W->I);
  const size_t need = moe::ffn_workspace_bytes(T, K, W->H, W->I, W->has_shared, act_mode);
  if (need > (size_t)MOE_NOALLOC_WS_BYTES)
    return fail(MOE_EWORKSPACE,
                "moe_expert_ffn_noalloc: these sizes need %zu bytes of workspace, more than the "
                "library's fixed %zu (use moe_expert_ffn with a caller workspace)",
                need, (size_t)MOE_NOALLOC_WS_BYTES);
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = moe::launch_expert_ffn(*W, x, T, K, offsets, sorted_slot, groups, act_mode, y_slots,
                             g_scratch[dev], (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_expert_ffn_noalloc launch");
}

int moe_route_permute(const float* logits, int T, int E, int K, int has_shared, int32_t* ids,
                      float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                      int32_t* slot_pos, int32_t* groups, void* ws, size_t ws_bytes,
                      void* stream) {
  if (!logits || !ids || !w || !counts || !offsets || !sorted_slot || !slot_pos || !groups)
    return fail(MOE_EINVAL, "moe_route_permute: null pointer");
  if (!sizes_ok_common(T, E, K) || (has_shared != 0 && has_shared != 1))
    return fail(MOE_EINVAL, "moe_route_permute: need T >= 1, 1 <= K <= min(E, 32), E <= 1024, has_shared in {0,1}");
  const size_t need = moe::permute_workspace_bytes(T, E, K);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_EWORKSPACE, "moe_route_permute: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  hipError_t e = moe::launch_route_permute(logits, T, E, K, has_shared, ids, w, counts, offsets,
                                           sorted_slot, slot_pos, groups, ws, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_route_permute launch");
}

int moe_expert_ffn_combine(const moe_nvfp4_weights* W, const uint16_t* x, int T, int K,
                           const int32_t* offsets, const int32_t* sorted_slot,
                           const int32_t* groups, int act_mode, const float* w,
                           const int32_t* slot_pos, const float* gate, uint16_t* y_slots,
                           uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !x || !offsets || !sorted_slot || !groups || !w || !slot_pos || !y_slots || !out)
    return fail(MOE_EINVAL, "moe_expert_ffn_combine: null pointer");
  if (!W->gu_codes || !W->gu_scales || !W->dn_codes || !W->dn_scales || !W->scale2)
    return fail(MOE_EINVAL, "moe_expert_ffn_combine: null weight pointer");
  if (act_mode < MOE_ACT_BF16 || act_mode > MOE_ACT_FP8_SHARED)
    return fail(MOE_EUNSUPPORTED, "moe_expert_ffn_combine: unknown act_mode %d", act_mode);
  if (!sizes_ok_common(T, W->E, K) || (W->has_shared != 0 && W->has_shared != 1))
    return fail(MOE_EINVAL, "moe_expert_ffn_combine: need T >= 1, 1 <= K <= min(E, 32), E <= 1024, has_shared in {0,1}");
  if (W->H < 256 || W->H > 4096 || W->H % 256 != 0 || W->I < 128 || W->I > 1024 || W->I % 128 != 0)
    return fail(MOE_EINVAL, "moe_expert_ffn_combine: need H a multiple of 256 in [256, 4096] and I a multiple of 128 in [128, 1024] (H=%d I=%d)", W->H, W->I);
  if (gate && !W->has_shared)
    return fail(MOE_EINVAL, "moe_expert_ffn_combine: a shared-expert gate needs has_shared");
  const size_t need = moe::ffn_combine_workspace_bytes(T, K, W->H, W->I, W->has_shared, act_mode);
  if (!ws || ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_expert_ffn_combine: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  hipError_t e = moe::launch_expert_ffn_combine(*W, x, T, K, offsets, sorted_slot, groups, act_mode,
                                                w, slot_pos, gate, y_slots, out, ws,
                                                (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_expert_ffn_combine launch");
}

int moe_layer(const moe_nvfp4_weights* W, const float* logits, const uint16_t* x, int T, int K,
              int act_mode, const float* gate, int32_t* ids, float* w, int32_t* counts,
              int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, int32_t* groups,
              uint16_t* y_slots, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !logits || !x || !ids || !w || !counts || !offsets || !sorted_slot || !slot_pos ||
      !groups || !y_slots || !out)
    return fail(MOE_EINVAL, "moe_layer: null pointer");
  if (!W->gu_codes || !W->gu_scales || !W->dn_codes || !W->dn_scales || !W->scale2)
    return fail(MOE_EINVAL, "moe_layer: null weight pointer");
  if (act_mode < MOE_ACT_BF16 || act_mode > MOE_ACT_FP8_SHARED)
    return fail(MOE_EUNSUPPORTED, "moe_layer: unknown act_mode %d", act_mode);
  if (!sizes_ok_common(T, W->E, K) || (W->has_shared != 0 && W->has_shared != 1))
    return fail(MOE_EINVAL, "moe_layer: need T >= 1, 1 <= K <= min(E, 32), E <= 1024, has_shared in {0,1}");
  if (W->H < 256 || W->H > 4096 || W->H % 256 != 0 || W->I < 128 || W->I > 1024 || W->I % 128 != 0)
    return fail(MOE_EINVAL, "moe_layer: need H a multiple of 256 in [256, 4096] and I a multiple of 128 in [128, 1024] (H=%d I=%d)", W->H, W->I);
  if (gate && !W->has_shared)
    return fail(MOE_EINVAL, "moe_layer: a shared-expert gate needs has_shared");
  const size_t need = moe::layer_workspace_bytes(T, W->E, K, W->H, W->I, W->has_shared, act_mode);
  if (!ws || ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_layer: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  const moe::RpOut ro{ids, w, counts, offsets, sorted_slot, slot_pos, groups};
  hipError_t e = moe::launch_layer(*W, logits, x, T, K, act_mode, gate, ro, y_slots, out, ws,
                                   (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_layer launch");
}

int moe_combine(const uint16_t* y_slots, const float* w, const int32_t* slot_pos, int T, int K,
                int H, int has_shared, uint16_t* out, void* stream) {
  if (!y_slots || !w || !slot_pos || !out) return fail(MOE_EINVAL, "moe_combine: null pointer");
  if (T < 1 || K < 1 || K > 32 || H < 8 || H % 8 != 0 || (has_shared != 0 && has_shared != 1) ||
      (long long)T * K > (1LL << 30))
    return fail(MOE_EINVAL, "moe_combine: need T >= 1, 1 <= K <= 32, H a positive multiple of 8, has_shared in {0,1}");
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  hipError_t e = moe::launch_combine(y_slots, w, slot_pos, nullptr, T, K, H, has_shared, out,
                                     (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_combine launch");
}

int moe_combine_gated(const uint16_t* y_slots, const float* w, const int32_t* slot_pos,
                      const float* gate, int T, int K, int H, uint16_t* out, void* stream) {
  if (!y_slots || !w || !slot_pos || !gate || !out)
    return fail(MOE_EINVAL, "moe_combine_gated: null pointer");
  if (T < 1 || K < 1 || K > 32 || H < 8 || H % 8 != 0 || (long long)T * K > (1LL << 30))
    return fail(MOE_EINVAL, "moe_combine_gated: need T >= 1, 1 <= K <= 32, H a positive multiple of 8");
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  hipError_t e = moe::launch_combine(y_slots, w, slot_pos, gate, T, K, H, 1, out, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_combine_gated launch");
}

int moe_router_topk(const moe_nvfp4_router* R, const uint16_t* x, int T, int K, int32_t* ids,
                    float* w, float* logits, float* gate, void* stream) {
  if (!R || !x || !ids || !w || !logits) return fail(MOE_EINVAL, "moe_router_topk: null pointer");
  if (!R->codes || !R->scales) return fail(MOE_EINVAL, "moe_router_topk: null weight pointer");
  if (R->has_gate != 0 && R->has_gate != 1)
    return fail(MOE_EINVAL, "moe_router_topk: has_gate must be 0 or 1");
  if (R->has_gate && !gate)
    return fail(MOE_EINVAL, "moe_router_topk: the matrix has a gate row but gate is NULL");
  if (!sizes_ok_common(T, R->E, K))
    return fail(MOE_EINVAL, "moe_router_topk: need T >= 1, 1 <= K <= min(E, 32), E <= 1024 (T=%d E=%d K=%d)", T, R->E, K);
  if (R->H < 256 || R->H > 8192 || R->H % 256 != 0 || (long long)T * R->H >= (1LL << 30))
    return fail(MOE_EINVAL, "moe_router_topk: need H a multiple of 256 in [256, 8192] and T*H < 2^30 (T=%d H=%d)", T, R->H);
  int rc = ensure_init();
  if (rc != MOE_OK) return rc;
  hipError_t e = moe::launch_router_topk(*R, x, T, K, ids, w, logits, R->has_gate ? gate : nullptr,
                                         (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "moe_router_topk launch");
}

int moe_timing_enable(int on) {
  g_timing_on.store(on != 0);
  return ok();
}

int moe_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_used = 0;
  g_dropped = 0;
  return ok();
}

int moe_timing_read(const char** names, int* launches, double* total_ms, int max_names,
                    int* dropped) {
  if (max_names < 0 || (max_names > 0 && (!names || !launches || !total_ms)))
    return fail(MOE_EINVAL, "moe_timing_read: bad output arrays");
  std::lock_guard<std::mutex> lk(g_tmu);
  int n = 0;
  for (size_t i = 0; i < g_used; ++i) {
    TimingRec& r = g_pool[i];
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "moe_timing_read: hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "moe_timing_read: hipEventElapsedTime");
    int j = 0;
    while (j < n && strcmp(names[j], r.name) != 0) ++j;
    if (j == n) {
      if (n == max_names) continue;
      names[n] = r.name;
      launches[n] = 0;
      total_ms[n] = 0.0;
      ++n;
    }
    launches[j] += 1;
    total_ms[j] += ms;
  }
  if (dropped) *dropped = (int)g_dropped;
  g_err.clear();
  return n;
}

}  // extern "C"
