"""Pins for the oracle's expert FFN and whole layer: closed forms built from
constant blocks (dim != inter so a transposed operand fails), clamps on and off,
zero input, one-hot routing, identical experts, shared-only, and the shape
checksum from the pages' parameter table."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import moe_ref as R
from synthetic import gen as G

D, I = 512, 256


def f16(v):
    return np.array([v], dtype=np.float16).view(np.uint8)


def const_q2k_matrix(rows, cols, a):
    """Every weight = a (sc = 1, q = 1, m = 0, d = a; a must be an fp16 value)."""
    blk = np.zeros(84, np.uint8)
    blk[0:16] = 0x01
    blk[16:80] = 0x55
    blk[80:82] = f16(a)
    return np.tile(blk, rows * cols // 256)


def const_q3k_matrix(rows, cols, w):
    """Every weight = w (q3 = 1: low 1 and high bit set; sc6 - 32 = 1; d = w)."""
    blk = np.zeros(110, np.uint8)
    blk[0:32] = 0xFF
    blk[32:96] = 0x55
    blk[96:104] = 0x11          # low nibbles of sc6 = 33 -> 1 for every sub-block
    blk[104:108] = 0xAA         # top pairs = 0b10 -> sc6 = 0b100001 = 33 for every sub-block
    blk[108:110] = f16(w)
    return np.tile(blk, rows * cols // 256)


def const_slot(a1, a3, w):
    return np.concatenate([const_q2k_matrix(I, D, a1), const_q2k_matrix(I, D, a3), const_q3k_matrix(D, I, w)])


def closed_form_expert(c, a1, a3, w, limit):
    """E(x = c everywhere) for constant-weight experts, from scalar arithmetic."""
    g = a1 * D * c
    u = a3 * D * c
    if limit > 0:
        g = min(g, limit)
        u = min(max(u, -limit), limit)
    h = np.float32(g / (1.0 + math.exp(-g)) * u)
    d = np.float32(abs(h)) / np.float32(127.0)
    hh = float(np.float16(d)) * 127.0 * (1 if h > 0 else -1)
    return w * I * hh


C = 127.0 / 128.0          # a bf16 value whose q8_1 is exact: d = 2^-7, q = 127


def bf16_bits_const(shape, v):
    return O.f32_to_bf16_bits(np.full(shape, v, dtype=np.float32))


@pytest.mark.parametrize("limit,a1,a3", [(10.0, 2.0 ** -10, -(2.0 ** -9)), (0.25, 2.0 ** -10, -(2.0 ** -9)),
                                         (0.25, -(2.0 ** -6), 2.0 ** -8), (0.0, 2.0 ** -5, 2.0 ** -6)])
def test_expert_closed_form(limit, a1, a3):
    cfg = R.MoeCfg(dim=D, inter=I, n_routed=1, topk=1, swiglu_limit=limit)
    w = 2.0 ** -8
    w1, w3, w2 = R.slot_matrices(cfg, const_slot(a1, a3, w))
    x = np.full((1, D), C, dtype=np.float32)
    e = R.expert_ffn_kquant(x, w1, w3, w2, limit)
    assert np.allclose(e, closed_form_expert(C, a1, a3, w, limit), rtol=1e-12, atol=0)


def test_swap_of_gate_and_up_is_visible():
    cfg = R.MoeCfg(dim=D, inter=I, n_routed=1, topk=1, swiglu_limit=10.0)
    w1, w3, w2 = R.slot_matrices(cfg, const_slot(2.0 ** -10, -(2.0 ** -9), 2.0 ** -8))
    x = np.full((1, D), C, dtype=np.float32)
    assert not np.allclose(R.expert_ffn_kquant(x, w1, w3, w2, 10.0), R.expert_ffn_kquant(x, w3, w1, w2, 10.0))


def bits(t):
    """bf16 torch tensor -> uint16 numpy bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def small_layer(n_routed=4, topk=1, seed=0):
    cfg = R.MoeCfg(dim=D, inter=I, n_routed=n_routed, topk=topk)
    shape = G.LayerShape(D, I, n_routed, topk)
    slots = [G.make_expert_slot(shape, seed, e).numpy() for e in range(n_routed)]
    wr, b = G.make_router(shape, seed, 0.05)
    return cfg, shape, slots, bits(wr), b.numpy()


def test_zero_input_gives_zero_output():
    cfg, shape, slots, wr, b = small_layer(n_routed=4, topk=2)
    sh = G.make_shared(shape, 0, "bf16")
    shared = {"fmt": "bf16", **{k: bits(sh[k]) for k in ("w1", "w3", "w2")}}
    out = R.moe_layer(cfg, np.zeros((3, D), np.uint16), wr, b, lambda e: slots[e], shared)
    assert np.all(out["y"] == 0.0)
    # with x = 0 every score is sqrt(ln 2): the selection follows the bias alone
    assert np.array_equal(out["idx"][0], np.argsort(-b, kind="stable")[:2])


def test_one_hot_routing_reproduces_single_expert():
    cfg, shape, slots, wr, b = small_layer(n_routed=4, topk=1)
    a1, a3, w = 2.0 ** -10, -(2.0 ** -9), 2.0 ** -8
    slots[2] = const_slot(a1, a3, w)
    b = np.zeros(4, np.float32)
    b[2] = 100.0
    x = bf16_bits_const((2, D), C)
    out = R.moe_layer(cfg, x, wr, b, lambda e: slots[e], None)
    assert np.all(out["idx"] == 2)
    s2 = out["s"][:, 2]
    expect = 1.5 * s2[:, None] * closed_form_expert(C, a1, a3, w, 10.0)
    assert np.allclose(out["y"], expect, rtol=1e-12, atol=0)


def test_identical_experts_sum_to_route_scale_times_one_expert():
    cfg, shape, slots, wr, b = small_layer(n_routed=4, topk=3)
    same = slots[1]
    x = bits(G.make_tokens(3, D, 7))
    out = R.moe_layer(cfg, x, wr, b, lambda e: same, None)
    w1, w3, w2 = R.slot_matrices(cfg, same)
    one = R.expert_ffn_kquant(O.bf16_bits_to_f64(x).astype(np.float32), w1, w3, w2, 10.0)
    assert np.allclose(out["y"], 1.5 * one, rtol=1e-12, atol=1e-15)


def test_shared_only_closed_form():
    cfg = R.MoeCfg(dim=D, inter=I, n_routed=2, topk=1)
    zero_slot = np.zeros(G.expert_layout(G.LayerShape(D, I, 2, 1))[0], np.uint8)   # d = 0 -> all weights 0
    wr = np.zeros((2, D), np.uint16)
    a1, a3, w = 2.0 ** -10, 2.0 ** -11, 2.0 ** -7
    shared = {"fmt": "bf16", "w1": bf16_bits_const((I, D), a1), "w3": bf16_bits_const((I, D), a3),
              "w2": bf16_bits_const((D, I), w)}
    x = bf16_bits_const((1, D), C)
    out = R.moe_layer(cfg, x, wr, np.zeros(2, np.float32), lambda e: zero_slot, shared)
    g, u = a1 * D * C, a3 * D * C
    h = np.float32(g / (1 + math.exp(-g)) * u)
    hb = float(O.bf16_bits_to_f64(O.f32_to_bf16_bits(h)))
    assert np.allclose(out["y"], w * I * hb, rtol=1e-13, atol=0)
    # K-quant shared with the same constant weights as a routed expert slot
    kq = {"fmt": "kquant", "slot": const_slot(2.0 ** -10, -(2.0 ** -9), 2.0 ** -8)}
    out = R.moe_layer(cfg, x, wr, np.zeros(2, np.float32), lambda e: zero_slot, kq)
    assert np.allclose(out["y"], closed_form_expert(C, 2.0 ** -10, -(2.0 ** -9), 2.0 ** -8, 10.0), rtol=1e-12)


def test_shape_checksum_against_parameter_table():
    # per routed expert 35,389,440 weights (3 x 5120 x 2304), 384 experts,
    # router 384 x 5120 (+ two 384-long bias vectors), total 13,626,901,248
    shape = G.REAL
    per_expert = 3 * shape.dim * shape.inter
    assert per_expert == 35_389_440
    router = shape.n_routed * shape.dim + 2 * shape.n_routed
    assert router == 1_966_848
    assert router + per_expert * (shape.n_routed + 1) == 13_626_901_248
    slot, o1, o3, o2 = G.expert_layout(shape)
    assert slot == 12_810_240 and o3 == 3_870_720 and o2 == 7_741_440
    assert (slot // 12_810_240) * per_expert == 35_389_440


def test_tolerance_rule():
    y = np.array([1.0, -0.5, 3.0])
    ok, ratio = R.within_tolerance(y + 2e-3 * 3.0 * 0.9, y)
    assert ok and ratio < 1
    ok, _ = R.within_tolerance(y + np.array([0, 0, 0.02]), y)   # bound at 3: 0.006 + ulp(3)/2 = 0.0138
    assert not ok
