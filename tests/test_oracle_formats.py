"""Pins for the oracle's number formats (bf16, fp16, Q2_K, Q3_K, q8_1).

The expected values here come from the format definitions and hand-built
blocks, not from the oracle: single-field probes state where each bit must land
(written as the inverse map, byte/bit -> weight index), closed forms give whole
blocks of known value, and constructed ties fix the rounding rules.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F

# ----------------------------------------------------------------------------- helpers

def f16_bytes(v):
    return np.array([v], dtype=np.float16).view(np.uint8)


def q2k_block(scales=None, qs=None, d=0.0, dmin=0.0):
    b = np.zeros(84, dtype=np.uint8)
    if scales is not None:
        b[0:16] = scales
    if qs is not None:
        b[16:80] = qs
    b[80:82] = f16_bytes(d)
    b[82:84] = f16_bytes(dmin)
    return b


def q3k_block(hmask=None, qs=None, scales12=None, d=0.0):
    b = np.zeros(110, dtype=np.uint8)
    if hmask is not None:
        b[0:32] = hmask
    if qs is not None:
        b[32:96] = qs
    if scales12 is not None:
        b[96:108] = scales12
    b[108:110] = f16_bytes(d)
    return b


def pack_q3k_scales(s6):
    """16 six-bit scales (0..63) -> 12 bytes, written from the byte-level rule:
    bytes 0..7 carry low nibbles (sub-blocks 0..7 low half, 8..15 high half),
    bytes 8..11 carry the 2-bit tops, four per byte."""
    out = np.zeros(12, dtype=np.uint8)
    for n, v in enumerate(s6):
        lo, hi = v & 15, v >> 4
        if n < 8:
            out[n] |= lo
        else:
            out[n - 8] |= lo << 4
        out[8 + n % 4] |= hi << (2 * (n // 4))
    return out


# ----------------------------------------------------------------------------- bf16 / fp16

def test_bf16_constructed_ties():
    u = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF, 0xBF818000], dtype=np.uint32)
    got = F.f32_to_bf16_bits(u.view(np.float32))
    assert list(got) == [0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF82]


def test_bf16_matches_torch_rne():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(100000) * np.exp2(rng.integers(-30, 30, 100000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16_bits(v), ref)


def test_bf16_decode_exact():
    assert list(F.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x4049]))) == [1.0, -2.0, 0.0, 3.140625]


def test_fp16_rne_ties_and_range():
    one = 1.0
    assert F.fp16_rne(np.float32(one + 2.0 ** -11)) == 1.0                    # tie -> even
    assert F.fp16_rne(np.float32(one + 3 * 2.0 ** -11)) == one + 2.0 ** -9     # tie -> even (up)
    assert F.fp16_rne(np.float32(65504.0)) == 65504.0
    assert F.fp16_rne(np.float32(2.0 ** -24)) == 2.0 ** -24                    # smallest subnormal


# ----------------------------------------------------------------------------- Q2_K

def test_q2k_sizes_and_offsets():
    assert F.Q2K_BYTES == 16 + 64 + 2 + 2 == 84
    blk = q2k_block(scales=np.full(16, 0x01, np.uint8), qs=np.full(64, 0xFF, np.uint8), d=2.0, dmin=0.0)
    assert np.all(F.dequant_q2k(blk) == 6.0)   # q = 3 everywhere, sc = 1, d = 2


@pytest.mark.parametrize("byte", range(64))
def test_q2k_single_field_probe(byte):
    # qs byte b = 32*h + l holds plane j at bits 2j..2j+1 for weight 128h + 32j + l
    h, l = divmod(byte, 32)
    for j in range(4):
        qs = np.zeros(64, np.uint8)
        qs[byte] = 2 << (2 * j)
        w = F.dequant_q2k(q2k_block(scales=np.full(16, 0x01, np.uint8), qs=qs, d=1.0))
        want = np.zeros(256)
        want[128 * h + 32 * j + l] = 2.0
        assert np.array_equal(w, want), (byte, j)


@pytest.mark.parametrize("n", range(16))
def test_q2k_scale_and_min_nibbles(n):
    # scale byte n drives exactly sub-block n (weights 16n..16n+15)
    scales = np.zeros(16, np.uint8)
    scales[n] = 0x5 | (0x3 << 4)
    w = F.dequant_q2k(q2k_block(scales=scales, qs=np.full(64, 0x55, np.uint8), d=0.5, dmin=0.25))
    want = np.zeros(256)
    want[16 * n:16 * n + 16] = 0.5 * 5 * 1 - 0.25 * 3
    assert np.array_equal(w, want)


def test_q2k_closed_forms():
    w = F.dequant_q2k(q2k_block(scales=np.full(16, 0x0F, np.uint8), qs=np.full(64, 0xFF, np.uint8), d=1.0))
    assert np.all(w == 45.0)
    w = F.dequant_q2k(q2k_block(scales=np.full(16, 0xF0, np.uint8), qs=np.zeros(64, np.uint8), dmin=1.0))
    assert np.all(w == -15.0)
    # sub-block ramp: sc_n = n, all q = 1 -> weight i = d * (i // 16)
    w = F.dequant_q2k(q2k_block(scales=np.arange(16, dtype=np.uint8), qs=np.full(64, 0x55, np.uint8), d=0.5))
    assert np.array_equal(w, 0.5 * (np.arange(256) // 16))


def test_q2k_loop_formulation_random():
    """A second, loop-shaped decoding of random blocks: walk the two 128-weight
    halves, the four bit planes and the two 16-weight runs of each plane."""
    rng = np.random.default_rng(1)
    for _ in range(20):
        blk = rng.integers(0, 256, 84, dtype=np.uint8)
        blk[80:82] = f16_bytes(rng.uniform(-1, 1))
        blk[82:84] = f16_bytes(rng.uniform(-1, 1))
        d = float(blk[80:82].view(np.float16)[0])
        dmin = float(blk[82:84].view(np.float16)[0])
        out, sub = [], 0
        for half in range(2):
            q = blk[16 + 32 * half:16 + 32 * half + 32]
            for plane in range(4):
                for run in range(2):
                    sc, mn = blk[sub] & 15, blk[sub] >> 4
                    sub += 1
                    for t in range(16):
                        out.append(d * sc * ((int(q[16 * run + t]) >> (2 * plane)) & 3) - dmin * mn)
        assert np.allclose(F.dequant_q2k(blk), out, rtol=0, atol=0)


# ----------------------------------------------------------------------------- Q3_K

def test_q3k_sizes():
    assert F.Q3K_BYTES == 32 + 64 + 12 + 2 == 110


@pytest.mark.parametrize("l", range(32))
def test_q3k_hmask_probe(l):
    # all low bits 0 and all high bits clear -> q3 = -4; setting bit b of hmask[l]
    # lifts weight 128*(b//4) + 32*(b%4) + l to q3 = 0
    s6 = pack_q3k_scales([33] * 16)           # sc6 - 32 = 1
    for bit in range(8):
        hm = np.zeros(32, np.uint8)
        hm[l] = 1 << bit
        w = F.dequant_q3k(q3k_block(hmask=hm, scales12=s6, d=1.0))
        want = np.full(256, -4.0)
        want[128 * (bit // 4) + 32 * (bit % 4) + l] = 0.0
        assert np.array_equal(w, want), (l, bit)


@pytest.mark.parametrize("n", range(16))
def test_q3k_scale_probe(n):
    # each of the 16 six-bit scales, probed through its low nibble and its top pair
    for val in (0x0B, 0x30, 0x3F, 0x00):
        s6 = [32] * 16                            # zero scale everywhere else
        s6[n] = val
        w = F.dequant_q3k(q3k_block(hmask=np.full(32, 0xFF, np.uint8), qs=np.full(64, 0x55, np.uint8),
                                    scales12=pack_q3k_scales(s6), d=0.5))
        want = np.zeros(256)
        want[16 * n:16 * n + 16] = 0.5 * (val - 32) * 1     # q3 = 1 (low 1, high set)
        assert np.array_equal(w, want), (n, val)


def test_q3k_extremes():
    # sc6 = 0 (scale -32) with q3 = -4 -> +128 d: the value an int8 fold cannot hold
    w = F.dequant_q3k(q3k_block(scales12=pack_q3k_scales([0] * 16), d=0.25))
    assert np.all(w == 128 * 0.25)
    # sc6 = 63 (scale +31) with q3 = 3 -> 93 d
    w = F.dequant_q3k(q3k_block(hmask=np.full(32, 0xFF, np.uint8), qs=np.full(64, 0xFF, np.uint8),
                                scales12=pack_q3k_scales([63] * 16), d=1.0))
    assert np.all(w == 93.0)


def test_q3k_loop_formulation_random():
    rng = np.random.default_rng(2)
    for _ in range(20):
        blk = rng.integers(0, 256, 110, dtype=np.uint8)
        blk[108:110] = f16_bytes(rng.uniform(-1, 1))
        d = float(blk[108:110].view(np.float16)[0])
        sc = blk[96:108]
        s6 = []
        for n in range(16):  # byte-level unpacking, written per sub-block
            lo = (sc[n] & 15) if n < 8 else (sc[n - 8] >> 4)
            hi = (sc[8 + n % 4] >> (2 * (n // 4))) & 3
            s6.append(int(lo | (hi << 4)) - 32)
        out, sub, bit = [], 0, 0
        for half in range(2):
            q = blk[32 + 32 * half:32 + 32 * half + 32]
            for plane in range(4):
                for run in range(2):
                    for t in range(16):
                        ll = 16 * run + t
                        lo2 = (int(q[ll]) >> (2 * plane)) & 3
                        hb = (int(blk[ll]) >> bit) & 1
                        out.append(d * s6[sub] * (lo2 - (0 if hb else 4)))
                    sub += 1
                bit += 1
        assert np.array_equal(F.dequant_q3k(blk), np.array(out))


# ----------------------------------------------------------------------------- q8_1

def test_q8_1_exact_multiples():
    k = np.arange(-127, 129, dtype=np.float64)[:256]
    k[k == 128] = 5
    c = 2.0 ** -7
    x = (c * k).astype(np.float32)
    q, d16, _ = F.quantize_q8_1(x)
    blocks = k.reshape(8, 32)
    amax = np.abs(blocks).max(axis=1)
    # d = amax*c/127; every block here holds exact multiples of its own d only when amax = 127
    for b in range(8):
        if amax[b] == 127:
            assert np.array_equal(q[32 * b:32 * b + 32], blocks[b].astype(np.int8))
            assert d16[b] == c


def test_q8_1_zero_block_and_extremes():
    x = np.zeros(64, np.float32)
    x[40] = -3.0
    x[41] = 1.5
    q, d16, s16 = F.quantize_q8_1(x)
    assert np.all(q[:32] == 0) and d16[0] == 0 and s16[0] == 0
    assert q[40] == -127
    assert q[41] == 64          # 1.5 / (3/127) = 63.5 -> away from zero


def test_q8_1_half_away_from_zero():
    x = np.zeros(32, np.float32)
    x[0] = 127.0            # d = 1 exactly
    x[1], x[2], x[3], x[4] = 2.5, -2.5, 0.5, -0.5
    q, d16, _ = F.quantize_q8_1(x)
    assert d16[0] == 1.0
    assert list(q[:5]) == [127, 3, -3, 1, -1]


def test_q8_1_values_use_fp16_scale():
    x = np.zeros(32, np.float32)
    x[0] = 1.0                                 # d = 1/127, not an fp16 value
    q, d16, _ = F.quantize_q8_1(x)
    assert q[0] == 127
    assert d16[0] == float(np.float16(np.float32(1.0) / np.float32(127.0)))
    assert F.q8_1_values(q, d16)[0] == 127 * d16[0]
