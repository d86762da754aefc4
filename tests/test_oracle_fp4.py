"""Pins for the oracle's MXFP4 decoder and its FP4 routed experts.

The expected values come from the format's definition, not from the oracle:
the eight e2m1 magnitudes and the E8M0 powers of two written out, one-nibble
and one-scale probes that state where each field must land, weights chosen
exactly representable so that the encode/decode round trip is exact, and a
closed-form expert with constant weights (dim != inter, so a transposed operand
fails).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import moe_ref as R
import synthetic as S
from synthetic import gen as G

# The e2m1 magnitudes of codes 0..7 (sign bit clear): 0, 0.5 (subnormal), then
# 1, 1.5, 2, 3, 4, 6 (exponents 0..2 with mantissa 0 or 1).
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def matrix_bytes(codes, scales):
    """codes int [rows, cols] (0..15), scales int [rows, cols/32] -> MXFP4 bytes."""
    codes = np.asarray(codes, dtype=np.uint8)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return np.concatenate([packed.reshape(-1), np.asarray(scales, dtype=np.uint8).reshape(-1)])


def test_e2m1_table():
    assert list(O.e2m1_value(np.arange(8))) == E2M1
    neg = O.e2m1_value(np.arange(8, 16))
    assert list(-neg) == E2M1
    assert math.copysign(1.0, neg[0]) == -1.0          # code 8 is -0


def test_e8m0_powers_of_two():
    assert O.e8m0_value(127) == 1.0
    assert O.e8m0_value(128) == 2.0
    assert O.e8m0_value(126) == 0.5
    assert O.e8m0_value(0) == 2.0 ** -127
    assert O.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(O.e8m0_value(255))


@pytest.mark.parametrize("col", [0, 1, 30, 31, 32, 63])
def test_one_nibble_probe(col):
    rows, cols = 2, 64
    codes = np.zeros((rows, cols), int)
    codes[1, col] = 5                                   # e2m1 3.0
    scales = np.full((rows, cols // 32), 127)
    w = O.dequant_mxfp4(matrix_bytes(codes, scales), rows, cols)
    expect = np.zeros((rows, cols))
    expect[1, col] = 3.0
    assert np.array_equal(w, expect)
    # the byte it lives in: low nibble for an even column, high for an odd one
    raw = matrix_bytes(codes, scales)
    byte = raw[1 * cols // 2 + col // 2]
    assert byte == (5 if col % 2 == 0 else 5 << 4)


@pytest.mark.parametrize("row,blk", [(0, 0), (0, 1), (2, 1), (2, 0)])
def test_one_scale_probe(row, blk):
    rows, cols = 3, 64
    codes = np.full((rows, cols), 1)                    # 0.5 everywhere
    scales = np.full((rows, cols // 32), 127)
    scales[row, blk] = 130                              # x8 for one block of one row
    raw = matrix_bytes(codes, scales)
    assert raw[rows * cols // 2 + row * (cols // 32) + blk] == 130    # scales follow all codes
    w = O.dequant_mxfp4(raw, rows, cols)
    expect = np.full((rows, cols), 0.5)
    expect[row, 32 * blk:32 * blk + 32] = 4.0
    assert np.array_equal(w, expect)


def test_representable_round_trip():
    rng = np.random.default_rng(7)
    rows, cols = 8, 256
    mags = rng.choice(E2M1, size=(rows, cols))
    mags[:, ::32] = 6.0                                 # every block reaches the largest magnitude
    sign = np.where(rng.random((rows, cols)) < 0.5, -1.0, 1.0)
    exps = rng.integers(-12, 3, size=(rows, cols // 32))
    w = sign * mags * np.repeat(np.exp2(exps.astype(np.float64)), 32, axis=1)
    raw = S.encode_mxfp4(torch.tensor(w, dtype=torch.float32)).numpy()
    assert raw.size == S.mxfp4_bytes(rows, cols)
    assert np.array_equal(O.dequant_mxfp4(raw, rows, cols), w)


D, I = 512, 256


def const_fp4_matrix(rows, cols, code, e):
    return matrix_bytes(np.full((rows, cols), code), np.full((rows, cols // 32), e))


@pytest.mark.parametrize("limit", [10.0, 0.25, 0.0])
def test_fp4_expert_closed_form(limit):
    # W1 = 1.5 * 2^-10 (code 3, E 117), W3 = -0.5 * 2^-8 (code 9, E 119), W2 = 2^-6 (code 2, E 121)
    a1, a3, w2v = 1.5 * 2.0 ** -10, -0.5 * 2.0 ** -8, 2.0 ** -6
    slot = np.concatenate([const_fp4_matrix(I, D, 3, 117), const_fp4_matrix(I, D, 9, 119),
                           const_fp4_matrix(D, I, 2, 121)])
    cfg = R.MoeCfg(dim=D, inter=I, n_routed=1, topk=1, swiglu_limit=limit, expert_fmt="fp4")
    w1, w3, w2 = R.slot_matrices(cfg, slot, "fp4")
    c = 0.75
    x = np.full((1, D), c)
    g, u = a1 * D * c, a3 * D * c
    if limit > 0:
        g = min(g, limit)
        u = min(max(u, -limit), limit)
    h = g / (1.0 + math.exp(-g)) * u
    hb = float(torch.tensor(h, dtype=torch.float32).to(torch.bfloat16).float())
    expect = w2v * I * hb
    e = R.shared_ffn_bf16(x, w1, w3, w2, limit)
    assert np.allclose(e, expect, rtol=1e-12, atol=0)


def test_fp4_layer_one_hot_routing():
    # one expert picked by every token (bias +100, k = 1): y = route_scale * s * E(x)
    shape = G.LayerShape(D, I, 3, 1)
    cfg = R.MoeCfg(dim=D, inter=I, n_routed=3, topk=1, expert_fmt="fp4")
    slots = [G.make_expert_slot(shape, 3, e, fmt="fp4").numpy() for e in range(3)]
    wr, _ = G.make_router(shape, 3, 0.05)
    bias = np.array([0.0, 100.0, 0.0], dtype=np.float32)
    x = G.make_tokens(2, D, 3)
    xb = x.contiguous().view(torch.int16).numpy().view(np.uint16)
    out = R.moe_layer(cfg, xb, wr.contiguous().view(torch.int16).numpy().view(np.uint16), bias,
                      lambda e: slots[e])
    assert (out["idx"] == 1).all()
    w1, w3, w2 = R.slot_matrices(cfg, slots[1], "fp4")
    xf = O.bf16_bits_to_f64(xb)
    e1 = R.shared_ffn_bf16(xf, w1, w3, w2, cfg.swiglu_limit)
    s = out["s"][np.arange(2), 1]
    assert np.allclose(out["y"], cfg.route_scale * s[:, None] * e1, rtol=1e-12, atol=1e-15)
    # and the FP4 weights are the encoder's input within half the largest e2m1 step
    # (2 x the block scale, which is below 2 amax / 6) of its block
    w1_draw = G.f32_normal((I, D), 0.02, G.stream_seed(3, G.TAG_EXPERT, 1, 0)).double().numpy()
    amax6 = np.repeat(np.max(np.abs(w1_draw.reshape(I, D // 32, 32)), axis=2) / 6.0, 32, axis=1)
    assert np.all(np.abs(w1 - w1_draw) <= 2.0 * amax6 + 1e-12)
