/*
 * moe_nvfp4.h -- C ABI of the routed mixture-of-experts FFN layer with NVFP4
 * weights and bf16 activations, for AMD Instinct MI355X (gfx950).
 *
 * One layer call is four entry points, run in this order on one HIP stream:
 *
 *   moe_route_topk  -> ids, w          router softmax + top-K per token
 *                                      (or moe_router_topk: router GEMM from
 *                                      NVFP4 weights fused with the top-K)
 *   moe_permute     -> counts, offsets, sorted_slot, slot_pos
 *   moe_expert_ffn  -> y_slots         gate_up GEMM, SiLU*up, down GEMM per
 *                                      expert group (routed + shared)
 *   moe_combine     -> out             fixed-order fp32 weighted sum
 *
 * Sources.  The operations are the ones listed as the prefill ops of a MoE
 * layer that can change the logits (router GEMM + top-k, shared expert, routed
 * experts, combine/unpermute) in the issue "[job] Qwen3.8-Flash-Next:
 * long-context cold prefill to SGLang parity"; the numerics (NVFP4 dequant as
 * e2m1 x e4m3 block scale x scale2, f32 accumulation, bf16 SiLU intermediate,
 * fp32 weighted combine) are the rows of that issue's table attributing the
 * transposed-MoE perplexity gap.  The tie rule of the router is the one of the
 * page "handover briefs" (item A1 and the indexer-selection kernel spec).
 *
 * Conventions for every entry point:
 *  - Every array pointer is a DEVICE pointer owned by the caller; the library
 *    keeps no reference after the call returns.  moe_nvfp4_weights is a host
 *    struct that holds device pointers.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  No entry point synchronises, allocates device memory,
 *    copies device to host or calls hipMemset, so a whole layer call can be
 *    captured into a HIP graph.
 *  - Return value: MOE_OK (0) or a negative status; moe_last_error() then
 *    holds a message for the calling thread.  Argument errors are detected on
 *    the host before anything is enqueued.  Faults inside a kernel surface at
 *    the caller's next synchronisation, as with any HIP kernel.
 *  - Integer stages are deterministic and bit-exact; floating stages use a
 *    fixed reduction order (no float atomics), so repeated calls on the same
 *    inputs give bitwise identical outputs.
 *
 * Limits: T >= 1, 1 <= K <= 32, K <= E <= 1024; for the expert FFN H is a
 * multiple of 256 in [256, 4096] and I a multiple of 128 in [128, 1024]; for
 * the combine H is a multiple of 8.  The library builds for gfx950
 * only; moe_init() refuses any other device.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK 0
#define MOE_EINVAL -1         /* null pointer, size out of range, bad combination */
#define MOE_EUNSUPPORTED -2   /* device is not gfx950, or unknown act_mode/op     */
#define MOE_EHIP -3           /* a HIP runtime call or kernel launch failed        */
#define MOE_EWORKSPACE -4     /* workspace smaller than moe_workspace_bytes()      */

/* Activation modes of moe_expert_ffn. */
#define MOE_ACT_BF16 0        /* gate_up reads the bf16 activations as they are    */
#define MOE_ACT_FP8_ROW 1     /* gate_up reads per-token-row e4m3 activations      */
#define MOE_ACT_FP8_ROUTED 2  /* routed experts e4m3, the shared expert bf16       */
#define MOE_ACT_FP8_SHARED 3  /* routed experts bf16, the shared expert e4m3       */

/* Operation ids of moe_workspace_bytes. */
#define MOE_OP_PERMUTE 1
#define MOE_OP_EXPERT_FFN 2
#define MOE_OP_EXPERT_FFN_COMBINE 3
#define MOE_OP_LAYER 4

/*
 * A bank of NVFP4 experts: E routed experts plus, if has_shared, one shared
 * expert at index E.  E' = E + has_shared groups, each laid out contiguously
 * (the resident [N, K/2] layout: one row per output feature, K contiguous):
 *
 *   gu_codes  [E'][2I][H/2]  e2m1 codes, two per byte, the low nibble is the
 *                            even K index; rows 0..I-1 = gate, I..2I-1 = up
 *   gu_scales [E'][2I][H/16] e4m3 (OCP "fn") scale of each 16 consecutive K
 *   dn_codes  [E'][H][I/2]
 *   dn_scales [E'][H][I/16]
 *   scale2    [E'][3]        fp32 per-tensor scale of gate, up, down
 *
 * Dequantised weight: W[n][k] = e2m1(code[n][k]) * e4m3(scale[n][k/16]) * scale2.
 */
typedef struct moe_nvfp4_weights {
  const uint8_t* gu_codes;
  const uint8_t* gu_scales;
  const uint8_t* dn_codes;
  const uint8_t* dn_scales;
  const float* scale2;
  int32_t E;
  int32_t H;
  int32_t I;
  int32_t has_shared;
} moe_nvfp4_weights;

/*
 * Check that the current HIP device is gfx950 and that every kernel of the
 * library is loadable (resolved once here, never per launch).  Returns MOE_OK,
 * MOE_EUNSUPPORTED (other architecture, the message names it) or MOE_EHIP.
 * The other entry points call it implicitly on first use per device.  The
 * refusing gate is the pages' convention for a single-architecture pilot: the
 * loader of the issue "EXL3 Qwen3.8-Flash-Next on CUDA sm_120 ...", section
 * "Scope: a pilot on sm_120", refuses any other compute capability with a
 * message that names the gate; here the gate is gfx950.
 */
int moe_init(void);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* moe_last_error(void);

/*
 * Device workspace, in bytes, that `op` needs for these sizes (0 if none).
 * Returns 0 for invalid sizes; the entry point itself reports the error.
 */
size_t moe_workspace_bytes(int op, int T, int E, int K, int H, int I, int has_shared,
                           int act_mode);

/*
 * Router top-K (the top-k of the router stage, the first prefill op of the
 * issue above's list; rank rule of the page "handover briefs", item A1 and the
 * indexer-selection kernel spec): for each token t, rank the E experts by logit (larger first,
 * equal logits -> lower index first, NaN counts as -inf), put the rank-k
 * expert in slot k, and weight the K selected experts by the softmax of their
 * logits: w[t][k] = exp(z_k - z_0) / sum_j exp(z_j - z_0), where a term with
 * z_k == z_0 is exp(0) = 1 even for infinite logits.  This equals the softmax
 * over all E experts restricted to the selected K and renormalised.
 *
 *   logits [T][E] float32, row-major      (in)
 *   ids    [T][K] int32                   (out) expert of each slot
 *   w      [T][K] float32                 (out) routing weight of each slot
 *
 * Limits: 1 <= K <= min(E, 32), E <= 1024.  Rows are independent.
 */
int moe_route_topk(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                   void* stream);

/*
 * An NVFP4 router matrix: R = E + has_gate rows of H, the same encoding as
 * the experts (listed as a w4a16 GEMM, 4-bit weights against 16-bit
 * activations, in the nsys kernel table of the issue "[job]
 * Qwen3.8-Flash-Next: long-context cold prefill to SGLang parity").  Rows
 * 0..E-1 give the expert logits; row E, when has_gate, gives the logit of the
 * shared expert's sigmoid gate.
 *
 *   codes  [R][H/2]   e2m1 codes, low nibble = even K index
 *   scales [R][H/16]  e4m3 scale of each 16 consecutive K
 *   scale2            fp32 scale of the whole matrix
 */
typedef struct moe_nvfp4_router {
  const uint8_t* codes;
  const uint8_t* scales;
  float scale2;
  int32_t E;
  int32_t H;
  int32_t has_gate;
} moe_nvfp4_router;

/*
 * Router gating GEMM fused with the top-K (the issue above names the router's
 * gating GEMM and its top-k as the first prefill op that moves the logits):
 *
 *   z[t][e] = scale2 * sum_k x[t][k] * e2m1(code[e][k]) * e4m3(scale[e][k/16])
 *
 * accumulated in f32 (order unspecified; |error| <= H * 2^-24 * sum_k |terms|),
 * then ids / w of each token exactly as moe_route_topk computes them from z
 * (two kernels: the GEMM writes z, the router's top-K reads it back).
 *
 *   R       host struct of device pointers, see moe_nvfp4_router
 *   x       [T][H] bf16 bit patterns                  (in)
 *   ids     [T][K] int32, w [T][K] float32            (out) as moe_route_topk
 *   logits  [T][E] float32                            (out) z
 *   gate    [T] float32 (required iff R->has_gate)    (out) row E's logit
 *
 * Limits: H a multiple of 256 in [256, 8192], 1 <= K <= min(E, 32),
 * E <= 1024, T * H < 2^30.  Rows are independent; the ids are those of
 * moe_route_topk applied to the returned logits, bit for bit.
 */
int moe_router_topk(const moe_nvfp4_router* R, const uint16_t* x, int T, int K, int32_t* ids,
                    float* w, float* logits, float* gate, void* stream);

/*
 * Group the T*K routed slots (slot s = t*K + k) by expert: the token
 * permutation, one of the per-layer MoE tensors that the prefill issue ("[job]
 * Qwen3.8-Flash-Next: long-context cold prefill to SGLang parity", section
 * "Localising the remaining ~0.56 %", the per-layer dump list) names between
 * the router's top-k ids/weights and the routed outputs before the combine.
 *
 *   ids         [T][K] int32, each in [0, E)   (in)
 *   counts      [E'] int32        (out) slots per group; counts[E] = T if shared
 *   offsets     [E'+1] int32      (out) exclusive prefix sum of counts
 *   sorted_slot [T*K + T*has_shared] int32 (out) slots grouped by expert, in
 *               ascending slot order inside each group; the shared group is
 *               slots T*K + t for t = 0..T-1 in token order, at positions
 *               offsets[E] + t (offsets[E] = T*K when every id is valid)
 *   slot_pos    [T*K + T*has_shared] int32 (out) position of slot s in
 *               sorted_slot, for the routed and the shared slots (the inverse)
 *   groups      [E'+1] int32      (out) groups[0] = number of non-empty
 *               groups; groups[1..groups[0]] = their indices, ascending;
 *               the remaining entries are -1
 *   ws          device workspace of at least
 *               moe_workspace_bytes(MOE_OP_PERMUTE, T, E, K, 0, 0, has_shared, 0)
 *
 * A slot whose id is outside [0, E) belongs to no group: it is not counted and
 * its slot_pos is -1 (later stages skip it).  The order never depends on
 * timing: positions are computed from counts, not from atomics.
 */
int moe_permute(const int32_t* ids, int T, int E, int K, int has_shared, int32_t* counts,
                int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, int32_t* groups,
                void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_topk followed by moe_permute, with the same outputs (ids, w and
 * the permutation arrays, bit for bit).  Batches of up to 8 tokens run as a
 * single kernel: one block routes them (a wave per token) and permutes the
 * ids from LDS, which takes a launch off the decode critical path; larger
 * batches run the two stages' own kernels.  ws: as moe_permute
 * (moe_workspace_bytes(MOE_OP_PERMUTE, ...)), NULL when that is 0.
 */
int moe_route_permute(const float* logits, int T, int E, int K, int has_shared, int32_t* ids,
                      float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                      int32_t* slot_pos, int32_t* groups, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * Expert FFN of every group on the rows routed to it.  For the row of sorted
 * position p in group e (token t = sorted_slot[p] / K, or sorted_slot[p] - T*K
 * in the shared group):
 *
 *   g = x[t] . W_gate,e^T,  u = x[t] . W_up,e^T          (f32 accumulate)
 *   h = bf16( silu(g) * u ),  silu(g) = g / (1 + exp(-g))
 *   y_slots[p] = bf16( h . W_down,e^T )
 *
 * with W the dequantised NVFP4 weights (scale2 applied to the f32 sums).
 * With act_mode MOE_ACT_FP8_ROW the gate_up input is instead the e4m3 row
 * quantisation of x: s_t = absmax(x[t]) / 448, q = e4m3_rne_sat(x[t] * (448 /
 * absmax)), and s_t multiplies the f32 sums of g and u (option (a) of the
 * issue above; weights stay exact, the e4m3 values enter the MFMA exactly).
 * MOE_ACT_FP8_ROUTED applies it to the routed experts only, the shared expert
 * reading the bf16 rows (arm S of the issue's shared-expert A/B table);
 * MOE_ACT_FP8_SHARED is the mirror (routed bf16, shared e4m3).
 *
 *   W        host struct of device pointers, see moe_nvfp4_weights
 *   x        [T][H] bf16 bit patterns                (in)
 *   offsets  [E'+1], sorted_slot [T*K + T*has_shared], groups [E'+1]
 *            from moe_permute (in)
 *   y_slots  [T*K + T*has_shared][H] bf16            (out) by sorted position
 *   ws       device workspace of at least
 *            moe_workspace_bytes(MOE_OP_EXPERT_FFN, T, E, K, H, I, has_shared, act_mode)
 *
 * T <= 8 runs the decode path (multi-row GEMV streaming each active expert's
 * weights once), larger T the grouped-GEMM path; both compute the same
 * function.  Rows whose sorted_slot entry is out of range are skipped.
 *
 * Workspace contents after the call (S = T*K + T*has_shared, A(n) = n rounded
 * up to a multiple of 256): bytes [0, 2*S*I) hold h as bf16 [S][I] by sorted
 * position; with MOE_ACT_FP8_ROW the e4m3 codes [T][H] follow at byte
 * A(2*S*I) and the fp32 row scales [T] at A(2*S*I) + A(T*H) (with the
 * per-class arms that region is scratch).  Scratch for the grouped path's
 * f16 activation rows ([T][H], [2T][H] with a per-class arm) and their fp32
 * epilogue factors comes next (its contents are unspecified after a call).
 */
int moe_expert_ffn(const moe_nvfp4_weights* W, const uint16_t* x, int T, int K,
                   const int32_t* offsets, const int32_t* sorted_slot, const int32_t* groups,
                   int act_mode, uint16_t* y_slots, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn followed by the combine (moe_combine, or moe_combine_gated
 * when `gate` is given) as one call, with the same y_slots and out.
 *
 *   w [T][K] float32, slot_pos [T*K + T*has_shared] int32   (in) routing
 *   gate [T] float32 or NULL (needs has_shared)              (in) shared gate logit
 *   y_slots, out                                            (out) as the two calls
 *   ws  at least moe_workspace_bytes(MOE_OP_EXPERT_FFN_COMBINE, ...) bytes,
 *       holding afterwards what moe_expert_ffn leaves in its workspace
 */
int moe_expert_ffn_combine(const moe_nvfp4_weights* W, const uint16_t* x, int T, int K,
                           const int32_t* offsets, const int32_t* sorted_slot,
                           const int32_t* groups, int act_mode, const float* w,
                           const int32_t* slot_pos, const float* gate, uint16_t* y_slots,
                           uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole layer in one call: moe_route_permute, then moe_expert_ffn_combine
 * (the layer's stages in the order of the issue "[job] Qwen3.8-Flash-Next:
 * long-context cold prefill to SGLang parity", section "Localising the
 * remaining ~0.56 %": router top-k, the permutation, the routed and shared
 * experts, the combine), with the same outputs bit for bit.  For decode
 * batches (T <= 8, the bf16 or the FP8 row arm, H / 128 in {2, 4, 8, 16} and
 * I / 128 in {1, 2, 4, 8}) it runs two or three kernels: every block of the
 * gate_up kernel routes and permutes the batch itself in LDS, so the routing
 * costs no launch of its own (the launch structure of the decode item A2 of
 * the page "handover briefs": top-10 + shared in one launch per projection);
 * then down and the combine, in one launch while at most 48 groups are
 * active.  Other calls run the route+permute and the FFN + combine kernels.
 *
 *   logits [T][E] float32                           (in)  router scores
 *   x, W, K, act_mode, gate                         (in)  as moe_expert_ffn_combine
 *   ids, w, counts, offsets, sorted_slot, slot_pos, groups
 *                                                   (out) as moe_route_permute
 *   y_slots, out                                    (out) as moe_expert_ffn_combine
 *   ws  at least moe_workspace_bytes(MOE_OP_LAYER, T, E, K, H, I, has_shared,
 *       act_mode) bytes (it serves the permutation, then the FFN)
 * Errors: those of the two calls, checked before anything is enqueued.
 */
int moe_layer(const moe_nvfp4_weights* W, const float* logits, const uint16_t* x, int T, int K,
              int act_mode, const float* gate, int32_t* ids, float* w, int32_t* counts,
              int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, int32_t* groups,
              uint16_t* y_slots, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and kernels as moe_expert_ffn, with the workspace taken from a
 * fixed array of MOE_NOALLOC_WS_BYTES inside the library (one per GPU,
 * resolved at moe_init and held until the process ends) instead of a caller
 * buffer.  The call allocates and frees nothing.
 *
 * Sizes whose moe_workspace_bytes(MOE_OP_EXPERT_FFN, ...) exceeds
 * MOE_NOALLOC_WS_BYTES return MOE_EWORKSPACE before anything is enqueued (at
 * H=2048, I=512, K=10 with a shared expert that is T > 2183 in the bf16 arm,
 * T > 1926 in the FP8 arm).  Every call on one GPU uses that GPU's single
 * array, so calls that overlap in time on one GPU (different streams, or
 * threads without ordering) race and must not be issued; calls ordered on one
 * stream are safe.  Nothing in the array needs to start at zero; its contents
 * after a call are those described for moe_expert_ffn's workspace.
 */
#define MOE_NOALLOC_WS_BYTES (32u << 20)
int moe_expert_ffn_noalloc(const moe_nvfp4_weights* W, const uint16_t* x, int T, int K,
                           const int32_t* offsets, const int32_t* sorted_slot,
                           const int32_t* groups, int act_mode, uint16_t* y_slots,
                           void* stream);

/*
 * Combine: out[t] = bf16( sum_{k=0..K-1} w[t][k] * y_slots[slot_pos[t*K+k]]
 *                          + y_slots[slot_pos[T*K + t]] (if has_shared) ),
 * accumulated in fp32 in exactly this order (slot order, then the shared
 * expert) with one round-to-nearest-even at the end, so the result does not
 * depend on how the work is split (the same-order rule of the issue "EXL3
 * Qwen3.8-Flash-Next on CUDA sm_120 ...", expert-parallel TP=2).
 *
 *   y_slots [T*K + T*has_shared][H] bf16, w [T][K] float32,
 *   slot_pos [T*K + T*has_shared] int32 from moe_permute  (in)
 *   out     [T][H] bf16 bit patterns  (out)
 *
 * Routed slots with slot_pos outside [0, T*K) and a shared slot outside
 * [0, T*K + T) are skipped.  H must be a multiple of 8.
 */
int moe_combine(const uint16_t* y_slots, const float* w, const int32_t* slot_pos, int T, int K,
                int H, int has_shared, uint16_t* out, void* stream);

/*
 * Combine with a gated shared expert: as moe_combine with has_shared = 1,
 * except that the shared expert's row is scaled by sigmoid(gate[t]) =
 * 1 / (1 + exp(-gate[t])) (fp32) before it is added:
 *
 *   out[t] = bf16( sum_k w[t][k] * y[slot_pos[t*K+k]] + sigmoid(gate[t]) * y[slot_pos[T*K+t]] )
 *
 * in that order.  gate [T] float32 is the router's row-E logit
 * (moe_router_topk's `gate`).  The pages name a shared expert next to the
 * routed ones but do not print its gate; this entry point covers the common
 * sigmoid-gated form, moe_combine the ungated one.
 */
int moe_combine_gated(const uint16_t* y_slots, const float* w, const int32_t* slot_pos,
                      const float* gate, int T, int K, int H, uint16_t* out, void* stream);

/*
 * Per-kernel timing, for measurement only.  While enabled, every kernel the
 * library launches is bracketed by two HIP events recorded on its stream (so
 * do not enable it while capturing a graph).  moe_timing_read() waits for the
 * recorded events and reports, for each kernel name launched since the last
 * reset, the number of launches and their summed duration in milliseconds.
 * At most 65536 launches are recorded between resets; later ones are counted
 * in `dropped`.  Returns the number of names written (<= max_names), or a
 * negative status.  Names are static strings owned by the library.
 */
int moe_timing_enable(int on);
int moe_timing_reset(void);
int moe_timing_read(const char** names, int* launches, double* total_ms, int max_names,
                    int* dropped);

#ifdef __cplusplus
}
#endif

#endif /* MOE_NVFP4_H */
