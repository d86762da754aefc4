"""The MoE feed-forward layer, written out plainly in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

What it computes, per token t (each step cites the passage it follows):
  1. router logits z = x W_R^T (Open Model Atlas, "DeepSeek V4.1 · Mixture of
     experts", router equation z = x_ffn W_R; metrale moe_v41 module doc:
     f32-accumulated router logits). Here: exact bf16 inputs, f64 sums.
  2. scores s = sqrt(softplus(z / gate_temp)), where softplus returns its
     argument above 20 (moe_v41.rs source view, fn ``softplus``; atlas router
     equation s = sqrt(softplus(z))).
  3. keys s + b; the top-k by key, descending, ties to the lower expert id, a
     NaN key is an error (moe_v41.rs, fn ``route_from_logits``: stable sort,
     "Panics on a NaN key").
  4. weights: the unbiased scores of the picks, divided by (sum + 1e-20) when
     norm_topk_prob and topk > 1, then times route_scale (``route_from_logits``;
     atlas equation G_i = 1.5 s_i / sum_j s_j).
  5. routed expert on the q8_1 activation: g = W1 x^, u = W3 x^, clamps
     g <= L and -L <= u <= L when L > 0, h = g sigma(g) u, then E = W2 q8_1(h)
     (atlas "Routed expert" equations; ``Expert.forward`` in the atlas' model.py
     excerpt for the clamp condition; moe_v41 module doc for q8_1 activations).
  5'. routed experts in MXFP4 (the upstream checkpoint's format; Open Model
     Atlas model.py excerpt: Expert with dtype float4_e2m1fn_x2): the same FFN
     on the unquantised bf16 x with the dequantised weights, h rounded to bf16
     before W2, as the excerpt's Linear layers compute in the activation dtype
     (the bf16 path of step 6).
  6. shared expert, added after the routed sum (atlas Delta_ffn = y_routed +
     y_shared; metrale ``shared_side``: added into acc after the routed
     experts). bf16 shared: unquantised x, h rounded to bf16 before W2 (the
     excerpt casts h back to the activation dtype); K-quant shared: step 5 with
     weight 1.
  7. y = sum_i G_i E_{T_i} + y_shared (atlas y_routed = sum G_i E_i), reported in
     f64 and rounded to bf16 (``bf16_bytes``).

Where the pages are silent: gate_temp = 1 and norm_topk_prob = true unless
given; the routing weight multiplies the expert output after W2; the q8_1
rounding is round-half-away-from-zero of x/d with the unrounded f32 d.

Pins (tests/test_oracle_layer.py, tests/test_oracle_route.py,
tests/test_oracle_matrices.py): brute-force top-k rank formulation on tiny
inputs, constructed ties, the sum-to-route_scale invariant, softplus closed
forms, closed-form experts (constant blocks), zero input, one-hot routing,
identical experts, shared-only; a slice of position-coded matrices decoded
into W1, W3, W2 in that order; the K-quant expert against a dense float64
expert on the decoded weights with unquantised activations (a hard error bound
and the RMS that the two q8_1 roundings predict).
"""

from dataclasses import dataclass

import numpy as np

from .formats import (
    FP4_BLOCK,
    Q2K_BYTES,
    Q3K_BYTES,
    QK_K,
    bf16_bits_to_f64,
    dequant_mxfp4,
    dequant_rows,
    f32_to_bf16_bits,
    q8_1_values,
    quantize_q8_1,
)


@dataclass
class MoeCfg:
    """Layer shape and routing constants (metrale ``MoeV41Cfg``)."""
    dim: int
    inter: int
    n_routed: int
    topk: int
    gate_temp: float = 1.0
    norm_topk_prob: bool = True
    route_scale: float = 1.5
    swiglu_limit: float = 10.0
    expert_fmt: str = "kquant"   # the routed experts: "kquant" (Q2_K/Q3_K) or "fp4" (MXFP4)


class NonFiniteKey(ValueError):
    """A routing key (score + bias) is NaN."""


# ----------------------------------------------------------------------------- routing

def router_logits(x, w_router):
    """z[t, e] = sum_d x[t, d] * W_R[e, d], float64."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T


def softplus_thresholded(v):
    """softplus(v) = v above 20, ln(1 + e^v) otherwise."""
    v = np.asarray(v, dtype=np.float64)
    safe = np.minimum(v, 20.0)
    return np.where(v > 20.0, v, np.log1p(np.exp(safe)))


def sqrt_softplus_scores(z, gate_temp):
    """s = sqrt(softplus(z / gate_temp))."""
    return np.sqrt(softplus_thresholded(np.asarray(z, dtype=np.float64) / gate_temp))


def select_topk(keys, k):
    """Indices of the k largest keys per row, in descending key order, equal keys
    ordered by ascending expert id. Raises NonFiniteKey on NaN."""
    keys = np.asarray(keys, dtype=np.float64)
    if np.isnan(keys).any():
        raise NonFiniteKey("NaN routing key")
    # a stable sort of the ids by descending key keeps equal keys in id order
    order = np.argsort(-keys, axis=-1, kind="stable")
    return order[..., :k]


def routing_weights(scores_picked, cfg):
    """Unbiased scores of the picks, renormalised when norm_topk_prob and
    topk > 1 (denominator sum + 1e-20), then times route_scale."""
    w = np.array(scores_picked, dtype=np.float64, copy=True)
    if cfg.norm_topk_prob and cfg.topk > 1:
        w = w / (w.sum(axis=-1, keepdims=True) + 1e-20)
    return w * cfg.route_scale


def route(cfg, x, w_router, bias):
    """Full routing for float64 inputs x [m, D]: returns (idx [m,k], G [m,k], keys [m,E], s [m,E])."""
    z = router_logits(x, w_router)
    s = sqrt_softplus_scores(z, cfg.gate_temp)
    keys = s + np.asarray(bias, dtype=np.float64)[None, :]
    idx = select_topk(keys, cfg.topk)
    g = routing_weights(np.take_along_axis(s, idx, axis=-1), cfg)
    return idx, g, keys, s


# ----------------------------------------------------------------------------- experts

def swiglu_clamped(g, u, limit):
    """h = min(g, L) * sigma(min(g, L)) * clip(u, -L, L); no clamping when L <= 0."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    if limit > 0:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    return g / (1.0 + np.exp(-g)) * u


def slot_matrices(cfg, raw, fmt="kquant"):
    """Decode one expert slice [W1 | W3 | W2] (W1/W3 [inter, dim], W2 [dim, inter])
    -> three float64 matrices. fmt "kquant": Q2_K, Q2_K, Q3_K blocks, rows in order;
    "fp4": three MXFP4 matrices."""
    raw = np.asarray(raw, dtype=np.uint8).reshape(-1)
    if fmt == "fp4":
        n13 = cfg.inter * cfg.dim // 2 + cfg.inter * cfg.dim // FP4_BLOCK
        n2 = cfg.dim * cfg.inter // 2 + cfg.dim * cfg.inter // FP4_BLOCK
        assert raw.size == 2 * n13 + n2, (raw.size, 2 * n13 + n2)
        return (dequant_mxfp4(raw[:n13], cfg.inter, cfg.dim), dequant_mxfp4(raw[n13:2 * n13], cfg.inter, cfg.dim),
                dequant_mxfp4(raw[2 * n13:], cfg.dim, cfg.inter))
    n13 = cfg.inter * (cfg.dim // QK_K) * Q2K_BYTES
    n2 = cfg.dim * (cfg.inter // QK_K) * Q3K_BYTES
    assert raw.size == 2 * n13 + n2, (raw.size, 2 * n13 + n2)
    w1 = dequant_rows(raw[:n13], cfg.inter, cfg.dim, "q2k")
    w3 = dequant_rows(raw[n13:2 * n13], cfg.inter, cfg.dim, "q2k")
    w2 = dequant_rows(raw[2 * n13:], cfg.dim, cfg.inter, "q3k")
    return w1, w3, w2


def q8_1_dequantized(x_f32):
    """x -> the values of its q8_1 quantisation (float64)."""
    q, d16, _ = quantize_q8_1(x_f32)
    return q8_1_values(q, d16)


def expert_ffn_kquant(x_f32, w1, w3, w2, limit):
    """One K-quant expert on f32 activations [T, dim]: q8_1(x), g/u, clamped
    SwiGLU, q8_1(f32(h)), then W2. Returns float64 [T, dim]."""
    xh = q8_1_dequantized(x_f32)
    g = xh @ w1.T
    u = xh @ w3.T
    h = swiglu_clamped(g, u, limit)
    hh = q8_1_dequantized(h.astype(np.float32))
    return hh @ w2.T


def shared_ffn_bf16(x, w1, w3, w2, limit):
    """bf16-activation expert (the bf16 shared expert; also a routed MXFP4 expert
    with its dequantised weights): unquantised x [T, dim] (float64 of bf16
    values), f64 g/u, clamped SwiGLU, h rounded to bf16 (through f32), then W2."""
    g = x @ w1.T
    u = x @ w3.T
    h = swiglu_clamped(g, u, limit)
    hb = bf16_bits_to_f64(f32_to_bf16_bits(h.astype(np.float32)))
    return hb @ w2.T


# ----------------------------------------------------------------------------- layer

def moe_layer(cfg, x_bits, router_bits, bias, expert_slot, shared=None):
    """The whole layer for m tokens.

    x_bits      uint16 [m, dim]        bf16 activations
    router_bits uint16 [n_routed, dim] bf16 router weight
    bias        float32 [n_routed]
    expert_slot callable e -> uint8 bytes of expert e's slice (see slot_matrices)
    shared      None, {"fmt": "bf16", "w1", "w3", "w2": uint16 bits} or
                {"fmt": "kquant", "slot": uint8 bytes}
    Returns dict(y float64 [m, dim], y_bf16 uint16 [m, dim], idx, G, keys, s).
    """
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    wr = bf16_bits_to_f64(np.asarray(router_bits, dtype=np.uint16))
    idx, gw, keys, s = route(cfg, x, wr, bias)
    m = x.shape[0]
    x32 = x.astype(np.float32)  # exact: every bf16 value is an f32 value
    # per-pick expert outputs, each expert decoded once for all tokens that picked it
    picks = np.zeros((m, cfg.topk, cfg.dim), dtype=np.float64)
    for e in np.unique(idx):
        w1, w3, w2 = slot_matrices(cfg, expert_slot(int(e)), cfg.expert_fmt)
        rows, cols = np.nonzero(idx == e)
        if cfg.expert_fmt == "fp4":
            picks[rows, cols] = shared_ffn_bf16(x[rows], w1, w3, w2, cfg.swiglu_limit)
        else:
            picks[rows, cols] = expert_ffn_kquant(x32[rows], w1, w3, w2, cfg.swiglu_limit)
    # routed sum in pick order, then the shared expert
    y = np.zeros((m, cfg.dim), dtype=np.float64)
    for i in range(cfg.topk):
        y += gw[:, i:i + 1] * picks[:, i, :]
    if shared is not None:
        if shared["fmt"] == "bf16":
            y += shared_ffn_bf16(
                x,
                bf16_bits_to_f64(shared["w1"]),
                bf16_bits_to_f64(shared["w3"]),
                bf16_bits_to_f64(shared["w2"]),
                cfg.swiglu_limit,
            )
        elif shared["fmt"] == "kquant":
            w1, w3, w2 = slot_matrices(cfg, shared["slot"])
            y += expert_ffn_kquant(x32, w1, w3, w2, cfg.swiglu_limit)
        else:
            raise ValueError(shared["fmt"])
    return {
        "y": y,
        "y_bf16": f32_to_bf16_bits(y.astype(np.float32)),
        "idx": idx,
        "G": gw,
        "keys": keys,
        "s": s,
    }


def ulp_bf16(v):
    """Spacing of bf16 numbers at |v|: 2^(floor(log2|v|) - 7); the smallest
    normal's spacing for zero."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    a = np.where(a == 0, np.finfo(np.float32).tiny, a)
    return np.exp2(np.floor(np.log2(a)) - 7)


def within_tolerance(gpu, ref):
    """The pass criterion: |gpu - y| <= 2e-3 * max|y| + ulp_bf16(y)/2 element-wise,
    against the unrounded float64 y. Returns (ok, worst_ratio)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = 2e-3 * np.max(np.abs(ref)) + 0.5 * ulp_bf16(ref)
    err = np.abs(gpu - ref)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    return bool(np.all(err <= bound)), ratio
