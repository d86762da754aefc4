"""Pins for the oracle's decoding of whole K-quant matrices and expert slices,
on data where every block differs.

The single-block pins (test_oracle_formats.py) fix where each bit of one
superblock lands. These fix the assembly above it, which tiles of identical
blocks cannot see: that row r of a matrix holds its cols/256 superblocks one
after another, rows in order (Q2_K for W1/W3 [inter, dim], Q3_K for W2
[dim, inter]), and that a slice is [W1 | W3 | W2].

  * Position-coded matrices (dim != inter): every block gets its own fp16 d
    (and dmin) from its row and superblock, its own random scales and quants.
    The blocks are packed here weight by weight from the byte/bit positions the
    GGUF layout gives each weight (the inverse of the decoder's map), and the
    expected matrix is written from the field values directly. A swapped row,
    a swapped superblock or a transposed block grid changes the values.
  * Encoder round trip on random f32 matrices: each decoded weight lies
    within one quantisation step of the f32 weight it was encoded from (a
    bound computed from the source sub-block alone, not from the bytes).
  * The K-quant expert against a dense float64 expert on the decoded weights
    with unquantised activations: the difference stays inside the error
    bound the two q8_1 steps allow, propagated through the products.
"""
import math

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe_ref as R
from synthetic import gen as G


def f16(v):
    return float(np.float16(v))


def f16_bytes(v):
    return np.array([v], dtype=np.float16).view(np.uint8)


# ----------------------------------------------------------------------------- block writers
# Weight i of a superblock (0..255): half h = i // 128, plane j = (i % 128) // 32,
# position l = i % 32, sub-block n = i // 16. The 2-bit field of weight i sits at
# bits 2j..2j+1 of qs byte 32h + l; the Q3_K high bit at bit 4h + j of hmask byte l.

def write_q2k(d, dmin, sc, mn, q):
    """One Q2_K block from its fields: d, dmin (fp16 values), sc[16], mn[16] (0..15),
    q[256] (0..3)."""
    b = np.zeros(84, np.uint8)
    for n in range(16):
        b[n] = int(sc[n]) | (int(mn[n]) << 4)
    for i in range(256):
        h, j, l = i // 128, (i % 128) // 32, i % 32
        b[16 + 32 * h + l] |= (int(q[i]) & 3) << (2 * j)
    b[80:82] = f16_bytes(d)
    b[82:84] = f16_bytes(dmin)
    return b


def write_q3k(d, s6, q3):
    """One Q3_K block: d (fp16 value), s6[16] six-bit scales (0..63), q3[256] in -4..3."""
    b = np.zeros(110, np.uint8)
    for i in range(256):
        h, j, l = i // 128, (i % 128) // 32, i % 32
        v = int(q3[i]) + 4                    # 0..7: low two bits, and the high bit set for q3 >= 0
        b[32 + 32 * h + l] |= (v & 3) << (2 * j)
        b[l] |= (v >> 2) << (4 * h + j)
    for n in range(16):
        lo, hi = s6[n] & 15, s6[n] >> 4
        if n < 8:
            b[96 + n] |= lo
        else:
            b[96 + n - 8] |= lo << 4
        b[96 + 8 + n % 4] |= hi << (2 * (n // 4))
    b[108:110] = f16_bytes(d)
    return b


def coded_q2k_matrix(rows, cols, seed):
    """Position-coded Q2_K matrix: (bytes, expected float64 [rows, cols])."""
    rng = np.random.default_rng(seed)
    nsb = cols // 256
    raw = np.zeros((rows, nsb, 84), np.uint8)
    want = np.zeros((rows, cols))
    for r in range(rows):
        for s in range(nsb):
            d = f16(2.0 ** -6 * (1 + r / 64.0 + s / 4096.0))       # distinct per (row, superblock)
            dmin = f16(2.0 ** -7 * (1 + s / 16.0 + r / 1024.0))
            sc = rng.integers(0, 16, 16)
            mn = rng.integers(0, 16, 16)
            q = rng.integers(0, 4, 256)
            raw[r, s] = write_q2k(d, dmin, sc, mn, q)
            for i in range(256):
                want[r, 256 * s + i] = d * sc[i // 16] * q[i] - dmin * mn[i // 16]
    return raw.reshape(-1), want


def coded_q3k_matrix(rows, cols, seed):
    rng = np.random.default_rng(seed)
    nsb = cols // 256
    raw = np.zeros((rows, nsb, 110), np.uint8)
    want = np.zeros((rows, cols))
    for r in range(rows):
        for s in range(nsb):
            d = f16(2.0 ** -8 * (1 + r / 64.0 + s / 4096.0))
            s6 = rng.integers(0, 64, 16)
            q3 = rng.integers(-4, 4, 256)
            raw[r, s] = write_q3k(d, s6, q3)
            for i in range(256):
                want[r, 256 * s + i] = d * (s6[i // 16] - 32) * q3[i]
    return raw.reshape(-1), want


DIM, INTER = 768, 512        # dim != inter, several superblocks per row both ways


@pytest.fixture(scope="module")
def coded():
    w1 = coded_q2k_matrix(INTER, DIM, 11)
    w3 = coded_q2k_matrix(INTER, DIM, 12)
    w2 = coded_q3k_matrix(DIM, INTER, 13)
    return w1, w3, w2


def test_position_coded_q2k_matrix(coded):
    raw, want = coded[0]
    got = F.dequant_rows(raw, INTER, DIM, "q2k")
    assert got.shape == (INTER, DIM)
    assert np.array_equal(got, want)


def test_position_coded_q3k_matrix(coded):
    raw, want = coded[2]
    got = F.dequant_rows(raw, DIM, INTER, "q3k")
    assert got.shape == (DIM, INTER)
    assert np.array_equal(got, want)


def test_position_coded_matrix_detects_reordering(coded):
    """The expected matrices are sensitive to every order the decoder could get
    wrong: two rows swapped, two superblocks of a row swapped, or the block grid
    read column-major."""
    raw, want = coded[0]
    blocks = raw.reshape(INTER, DIM // 256, 84)
    rows_swapped = blocks.copy()
    rows_swapped[[3, 4]] = rows_swapped[[4, 3]]
    sb_swapped = blocks.copy()
    sb_swapped[5, [0, 2]] = sb_swapped[5, [2, 0]]
    col_major = blocks.transpose(1, 0, 2).copy()
    for bad in (rows_swapped, sb_swapped, col_major):
        assert not np.array_equal(F.dequant_rows(bad.reshape(-1), INTER, DIM, "q2k"), want)


def test_slot_is_w1_w3_w2_in_that_order(coded):
    (r1, e1), (r3, e3), (r2, e2) = coded
    cfg = R.MoeCfg(dim=DIM, inter=INTER, n_routed=1, topk=1)
    slot = np.concatenate([r1, r3, r2])
    size, o1, o3, o2 = G.expert_layout(G.LayerShape(DIM, INTER, 1, 1))
    assert slot.size == size and (o1, o3, o2) == (0, r1.size, 2 * r1.size)
    w1, w3, w2 = R.slot_matrices(cfg, slot)
    assert np.array_equal(w1, e1) and np.array_equal(w3, e3) and np.array_equal(w2, e2)


# ----------------------------------------------------------------------------- encoder round trip

def _subblocks(w):
    rows, cols = w.shape
    return w.reshape(rows * cols // 256, 16, 16).astype(np.float64)


def q2k_step_bound(w):
    """Per weight: a bound on |decoded - source| for the min/max encoder, from the
    source sub-block alone. step = (max - min(0, min)) / 3 is the spacing of the
    four levels; the stored scale and min are 4-bit multiples of d and dmin
    (the largest step / 15 and largest -min / 15 of the superblock), so each is
    off by at most half of d or dmin (plus fp16 rounding of d and dmin), and the
    top level can fall short of max by three times the scale's error."""
    x = _subblocks(w)
    lo = np.minimum(0.0, x.min(-1))
    step = (x.max(-1) - lo) / 3.0
    d = step.max(-1, keepdims=True) / 15.0 * (1 + 2.0 ** -10)
    dmin = (-lo).max(-1, keepdims=True) / 15.0 * (1 + 2.0 ** -10)
    b = np.maximum(0.5 * (step + 0.5 * d), 1.5 * d + 0.5 * dmin) + 0.5 * dmin
    return np.repeat(b[..., None], 16, -1).reshape(w.shape)


def q3k_step_bound(w):
    """Per weight: the min/max Q3_K encoder maps the sub-block's signed value of
    largest magnitude to q3 = -4, so the unit is about |amax| / 4 (a 6-bit
    multiple of d = largest unit / 32, off by at most d / 2); values at the
    opposite end clamp to q3 = 3, one unit short, so one unit plus four times
    the scale's error bounds the difference."""
    x = _subblocks(w)
    unit = np.abs(x).max(-1) / 4.0
    d = unit.max(-1, keepdims=True) / 32.0 * (1 + 2.0 ** -10)
    b = unit + 0.5 * d + 4 * 0.5 * d
    return np.repeat(b[..., None], 16, -1).reshape(w.shape)


@pytest.mark.parametrize("rows,cols,std", [(40, 768, 0.02), (16, 512, 1.0), (24, 256, 3e-4)])
def test_encoder_round_trip_q2k(rows, cols, std):
    w = G.f32_normal((rows, cols), std, 100 + rows).numpy()
    raw = G.encode_q2k(torch.from_numpy(w)).numpy().reshape(-1)
    got = F.dequant_rows(raw, rows, cols, "q2k")
    bound = q2k_step_bound(w)
    err = np.abs(got - w.astype(np.float64))
    assert np.all(err <= bound), float(np.max(err / bound))
    # the bound is not loose: on average a weight is much closer than it
    assert err.mean() < 0.4 * bound.mean()
    # and decoding the rows in another order breaks it
    bad = raw.reshape(rows, -1)[::-1].reshape(-1)
    assert not np.all(np.abs(F.dequant_rows(bad, rows, cols, "q2k") - w) <= bound)


@pytest.mark.parametrize("rows,cols,std", [(40, 512, 0.02), (8, 768, 1.0), (16, 256, 5e-4)])
def test_encoder_round_trip_q3k(rows, cols, std):
    w = G.f32_normal((rows, cols), std, 200 + rows).numpy()
    raw = G.encode_q3k(torch.from_numpy(w)).numpy().reshape(-1)
    got = F.dequant_rows(raw, rows, cols, "q3k")
    bound = q3k_step_bound(w)
    err = np.abs(got - w.astype(np.float64))
    assert np.all(err <= bound), float(np.max(err / bound))
    assert err.mean() < 0.4 * bound.mean()
    bad = raw.reshape(rows, cols // 256, 110)[:, ::-1].reshape(-1)   # superblocks of each row reversed
    if cols > 256:
        assert not np.all(np.abs(F.dequant_rows(bad, rows, cols, "q3k") - w) <= bound)


# ----------------------------------------------------------------------------- expert vs dense f64

def q8_1_error_bound(v):
    """Per element: |q8_1 value - v| <= d/2 + 127 * |fp16(d) - d|, with
    d = amax / 127 of the element's 32-block and the fp16 rounding of d at most
    2^-11 d (normal range)."""
    v = np.asarray(v, np.float64)
    blk = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    d = np.abs(blk).max(-1, keepdims=True) / 127.0
    b = (0.5 * d + 127 * 2.0 ** -11 * d) * (1 + 1e-6)
    return np.broadcast_to(b, blk.shape).reshape(v.shape)


def swiglu_slopes(g, u, limit):
    """|dh/dg| and |dh/du| of the clamped SwiGLU at (g, u); zero where a clamp
    holds the input."""
    gc = np.minimum(g, limit) if limit > 0 else g
    uc = np.clip(u, -limit, limit) if limit > 0 else u
    sig = 1.0 / (1.0 + np.exp(-gc))
    dg = np.abs(sig * (1 + gc * (1 - sig)) * uc)      # d/dg of g sigma(g) u; |sigma (1 + g (1 - sigma))| <= 1.1
    du = np.abs(gc * sig)
    if limit > 0:
        dg = np.where(g > limit, 0.0, dg)
        du = np.where(np.abs(u) > limit, 0.0, du)
    return dg, du


def q8_1_step(v):
    """Per element: the q8_1 step d = amax / 127 of its 32-block."""
    v = np.asarray(v, np.float64)
    blk = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    d = np.abs(blk).max(-1, keepdims=True) / 127.0
    return np.broadcast_to(d, blk.shape).reshape(v.shape)


@pytest.mark.parametrize("limit,xstd", [(10.0, 1.0), (0.25, 1.0), (0.0, 3.0)])
def test_kquant_expert_against_dense_product(limit, xstd):
    """E(x) of the oracle (q8_1 of x, q8_1 of h) against W2 h(W1 x, W3 x) in
    float64 on the same decoded weights with nothing quantised.

    Two statements about the difference:
      * a hard bound: the worst-case q8_1 error of x carried through |W1|, |W3|
        and the SwiGLU slopes, plus the q8_1 error of h, carried through |W2|
        (first order, doubled to cover the second-order terms);
      * its size: rounding to a q8_1 grid errs like a uniform variable of
        variance d^2 / 12, so the propagated variance predicts the RMS of the
        difference. The measured RMS must match it within a factor of 4/3;
        leaving out either quantisation, or a wrong operand, moves it out.
    """
    shape = G.LayerShape(DIM, INTER, 1, 1)
    cfg = R.MoeCfg(dim=DIM, inter=INTER, n_routed=1, topk=1, swiglu_limit=limit)
    slot = G.make_expert_slot(shape, 3, 0, std=0.05).numpy()
    w1, w3, w2 = R.slot_matrices(cfg, slot)
    x = G.f32_normal((5, DIM), xstd, 77).numpy()
    got = R.expert_ffn_kquant(x, w1, w3, w2, limit)

    xd = x.astype(np.float64)
    g = xd @ w1.T
    u = xd @ w3.T
    gc = np.minimum(g, limit) if limit > 0 else g
    uc = np.clip(u, -limit, limit) if limit > 0 else u
    h = gc / (1 + np.exp(-gc)) * uc
    dense = h @ w2.T
    diff = got - dense
    sg, su = swiglu_slopes(g, u, limit)

    ex = q8_1_error_bound(x)
    eg = ex @ np.abs(w1).T
    eu = ex @ np.abs(w3).T
    eh = 2.0 * (1.1 * np.abs(uc) * eg + np.abs(gc) * eu + eg * eu)
    eh = eh + q8_1_error_bound(np.abs(h) + eh)
    bound = 2.0 * (eh @ np.abs(w2).T)
    assert np.all(np.abs(diff) <= bound), float(np.max(np.abs(diff) / bound))

    vx = q8_1_step(xd) ** 2 / 12
    vh = sg ** 2 * (vx @ (w1 ** 2).T) + su ** 2 * (vx @ (w3 ** 2).T) + q8_1_step(h) ** 2 / 12
    predicted = math.sqrt(float((vh @ (w2 ** 2).T).mean()))
    rms = math.sqrt(float((diff ** 2).mean()))
    assert 0.75 * predicted <= rms <= 1.33 * predicted, (rms, predicted)
    # gate and up exchanged: far outside
    swapped = R.expert_ffn_kquant(x, w3, w1, w2, limit) - dense
    assert math.sqrt(float((swapped ** 2).mean())) > 10 * predicted
