"""Seeded synthetic inputs for the MoE layer: the only module both the HIP path's
tests/benchmark and the CPU oracle draw from.

It holds none of the layer's arithmetic (no routing, no dot products, no
activation quantisation). It draws weights and tokens from seeded generators
and packs weight draws into GGUF Q2_K / Q3_K blocks with a simple min/max
encoder, or into microscaled FP4 (e2m1 codes, E8M0 scales per 32 weights);
those encoders are test-data preparation (the pages' experts arrive already
quantised), and the layer only ever decodes the bytes they produce.
"""

from .gen import (  # noqa: F401
    LayerShape,
    TINY,
    REAL,
    stream_seed,
    bf16_normal,
    uniform_f32,
    encode_q2k,
    encode_q3k,
    encode_mxfp4,
    mxfp4_bytes,
    FP4_BLOCK,
    expert_layout,
    make_expert_slot,
    make_experts,
    random_kquant_slot,
    make_router,
    make_shared,
    make_tokens,
    skewed_bias,
    C4_BIAS_SCALE,
)
