"""Plain float64 CPU oracle for the DeepSeek-V4.1-style quantised MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY. Nothing here is part of the product path: only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it. It shares no code with the HIP library (no kernels, headers,
tables or helpers); the only thing both sides use is the seeded input generator
package ``synthetic``, which holds none of the layer's arithmetic.

Sources (the pages this is written from):
  * metrale ``moe_v41`` module documentation and its ``moe_v41.rs`` source view
    (docs.metrale.ai): routing semantics of ``route_from_logits``, the
    thresholded ``softplus``, ``bf16_bytes``, ``MoeV41Cfg``.
  * Open Model Atlas, "DeepSeek V4.1 · Mixture of experts": the router and
    expert equations ("All 22 steps"), the ``Gate``/``Expert``/``MoE`` code
    excerpts and ``config.json``.
The Q2_K / Q3_K / q8_1 byte layouts are not printed on the pages (they only
name the formats); they follow the public GGUF K-quant block format. The
MXFP4 scale layout is not printed either (the pages give the e2m1 element type
of the upstream experts); it follows the OCP microscaling format.

Parity status per function is stated in each module's header.
"""

from .formats import (  # noqa: F401
    QK_K,
    Q2K_BYTES,
    Q3K_BYTES,
    bf16_bits_to_f64,
    f32_to_bf16_bits,
    fp16_rne,
    dequant_q2k,
    dequant_q3k,
    FP4_BLOCK,
    e2m1_value,
    e8m0_value,
    dequant_mxfp4,
    quantize_q8_1,
    q8_1_values,
)
from .moe_ref import (  # noqa: F401
    MoeCfg,
    NonFiniteKey,
    router_logits,
    softplus_thresholded,
    sqrt_softplus_scores,
    select_topk,
    routing_weights,
    route,
    swiglu_clamped,
    expert_ffn_kquant,
    shared_ffn_bf16,
    slot_matrices,
    moe_layer,
    ulp_bf16,
    within_tolerance,
)
