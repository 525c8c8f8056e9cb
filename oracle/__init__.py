"""Plain fp64 CPU oracle for the NVFP4 routed-MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
anything in this package: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers); both sides only take their
inputs from the seeded generators in ``workloads``.

Sources (the web pages this layer is described on):

* [attr]   issue "[job] Qwen3.8-Flash-Next: long-context cold prefill to SGLang
           parity", the table that attributes the transposed-MoE perplexity gap
           (rows: activations into the MMA, weights, accumulation/SiLU/combine).
* [opts]   same issue, options (a) per-token-row e4m3 activation scale, (b), (c).
* [local]  same issue, the list of prefill ops that can change logits (router
           GEMM + top-k, shared expert, routed experts, combine/unpermute) and
           the per-layer dump list (logits, top-k ids/weights, permutation, ...).
* [job]    same issue, "What's the job?": the resident [N, K/2] NVFP4 layout.
* [A1]     page "handover briefs", item A1 subtask 1: top-k with torch's
           tie-break, the lower index wins on equal score.
* [topk]   same page, the device-side indexer selection kernel spec: rank of b is
           the count of j with s_j > s_b or (s_j == s_b and j < b); NaN = -inf.
* [A2]     same page, item A2 (MoE decode: gate+up fused, silu+down fused,
           top-10 experts and the shared expert).
* [tp2]    issue "EXL3 Qwen3.8-Flash-Next on CUDA sm_120: expert offload, TP=2,
           graphs and MTP", section on expert offload: per-slot expert outputs
           summed in the same order as one rank; Questions item 2.
* [nsys]   same issue, the per-kernel table of the prefill profile: the router
           runs as a w4a16 GEMM.
* [fp4local] same issue, the FP4-Local section: the only dequant kernel left is
           the router dequant.
* [OCP]    the OCP Microscaling Formats (MX) v1.0 and OCP 8-bit floating point
           specifications, which define the e2m1 and e4m3 ("fn") encodings the
           pages name.

Parity status of every function is listed in its module header.
"""
from .formats import (  # noqa: F401
    e2m1_decode,
    e4m3_decode,
    unpack_nibbles,
    dequant_nvfp4,
    e4m3_encode_rne_sat,
    E4M3_MAX,
)
from .route import route_topk  # noqa: F401
from .permute import permute  # noqa: F401
from .ffn import silu, expert_ffn, expert_outputs, combine, moe_layer  # noqa: F401
from .fp8 import rowquant_e4m3, rowquant_dequant  # noqa: F401
from .router import router_logits, router_route, sigmoid  # noqa: F401
