"""Number formats of the MoE layer, decoded plainly in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

Formats:
  * bf16: round-to-nearest-even from f32, as metrale's ``bf16_bytes`` states it
    (moe_v41.rs source view, fn ``bf16_bytes``: add 0x7FFF plus the lowest kept
    bit, keep the high half).
  * fp16: IEEE binary16, round to nearest even.
  * Q2_K / Q3_K: 256-weight GGUF K-quant superblocks. The pages only name them
    (moe_v41 module documentation: gate/up on Q2_K kernels, down on Q3_K); the
    layouts below are the public GGUF ones, restated here in our own words.
  * q8_1: 32-value blocks of int8 with an fp16 scale d and fp16 d*sum (named on
    the pages: "the activation quantised to q8_1").
  * MXFP4: the routed experts' own format upstream (Open Model Atlas, "DeepSeek
    V4.1 · Mixture of experts": the experts are stored as float4_e2m1fn_x2, two
    FP4 values per byte, in the model.py excerpt and config.json expert_dtype
    "fp4"). The pages give the element type only; the scale layout read here is
    the OCP microscaling one: per 32 consecutive weights of a row one E8M0
    scale 2^(E-127); each weight an e2m1 code (sign bit 3, two exponent bits with
    bias 1, one mantissa bit), the even weight of a pair in the low nibble. A
    matrix is its codes [rows, cols/2] followed by its scales [rows, cols/32].

Pins (tests/test_oracle_formats.py): single-field probes and closed forms for
both block decoders, constructed rounding ties, q8_1 closed forms; for MXFP4
the eight e2m1 magnitudes against the format's definition, E8M0 powers of two,
one-nibble and one-scale probes, and exactly representable matrices.
Whole K-quant matrices (tests/test_oracle_matrices.py): position-coded matrices
whose every block has its own d, dmin, scales and quants, packed weight by
weight from the layout and compared value for value (row order, superblock
order, orientation); the encoder round trip within one quantisation step.
"""

import numpy as np

QK_K = 256          # weights per K-quant superblock
Q2K_BYTES = 84      # scales[16] | qs[64] | d fp16 | dmin fp16
Q3K_BYTES = 110     # hmask[32] | qs[64] | scales[12] | d fp16
Q8_BLOCK = 32       # values per q8_1 block


# ----------------------------------------------------------------------------- bf16 / fp16

def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(v):
    """f32 -> bf16 bits, nearest with ties to even (metrale ``bf16_bytes`` rule)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return (((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)).astype(np.uint16)


def fp16_rne(v):
    """Round float32 values to IEEE binary16 (nearest even); returned as float64."""
    return np.asarray(v, dtype=np.float32).astype(np.float16).astype(np.float64)


def _fp16_field(blocks, offset):
    """Little-endian fp16 stored at byte ``offset`` of each block -> float64."""
    raw = np.ascontiguousarray(blocks[..., offset:offset + 2])
    return raw.view(np.float16)[..., 0].astype(np.float64)


# ----------------------------------------------------------------------------- weight index map
# Superblock weight i (0..255): half h = i // 128, r = i % 128, 2-bit plane j = r // 32,
# position l = r % 32; sub-block n = i // 16 (16 sub-blocks of 16 weights).

_I = np.arange(QK_K)
_H = _I // 128
_J = (_I % 128) // 32
_L = _I % 32
_N = _I // 16


def dequant_q2k(blocks):
    """Q2_K superblocks uint8[..., 84] -> float64[..., 256].

    Layout: bytes 0..15 scales (low nibble sc_n, high nibble m_n for sub-block n),
    bytes 16..79 qs (2-bit quants, four planes per byte), 80..81 d, 82..83 dmin.
    Weight i = d * sc_n * q_i - dmin * m_n with q_i = (qs[32h + l] >> 2j) & 3.
    """
    b = np.asarray(blocks, dtype=np.uint8)
    assert b.shape[-1] == Q2K_BYTES
    scales = b[..., 0:16].astype(np.int64)
    qs = b[..., 16:80].astype(np.int64)
    d = _fp16_field(b, 80)
    dmin = _fp16_field(b, 82)
    q = (qs[..., 32 * _H + _L] >> (2 * _J)) & 3
    sc = scales[..., _N] & 15
    mn = scales[..., _N] >> 4
    return d[..., None] * sc * q - dmin[..., None] * mn


def q3k_scale6(scales12, n):
    """The signed 6-bit scale (sc6 - 32) of sub-block n from the 12 packed scale bytes.

    Low 4 bits: sub-blocks 0..7 use the low nibble of byte n, 8..15 the high
    nibble of byte n-8. High 2 bits: bits 2*(n//4)..+1 of byte 8 + n%4.
    """
    s = np.asarray(scales12).astype(np.int64)
    n = np.asarray(n)
    low4 = np.where(n < 8, s[..., n % 8] & 15, s[..., n % 8] >> 4)
    hi2 = (s[..., 8 + n % 4] >> (2 * (n // 4))) & 3
    return (low4 | (hi2 << 4)) - 32


def dequant_q3k(blocks):
    """Q3_K superblocks uint8[..., 110] -> float64[..., 256].

    Layout: bytes 0..31 hmask (high bit of weight i is bit 4h+j of hmask[l]),
    32..95 qs (low 2 bits, same plane layout as Q2_K), 96..107 packed 6-bit
    scales, 108..109 d. q3 = low - (4 if the high bit is clear else 0), in
    [-4, 3]; weight i = d * (sc6_n - 32) * q3_i.
    """
    b = np.asarray(blocks, dtype=np.uint8)
    assert b.shape[-1] == Q3K_BYTES
    hmask = b[..., 0:32].astype(np.int64)
    qs = b[..., 32:96].astype(np.int64)
    scales = b[..., 96:108]
    d = _fp16_field(b, 108)
    low = (qs[..., 32 * _H + _L] >> (2 * _J)) & 3
    high = (hmask[..., _L] >> (4 * _H + _J)) & 1
    q3 = low - np.where(high == 1, 0, 4)
    s6 = q3k_scale6(scales, _N)
    return d[..., None] * s6 * q3


def dequant_rows(raw, n_rows, n_cols, kind):
    """A row-major matrix of K-quant blocks (bytes) -> float64 [n_rows, n_cols]."""
    nb = n_cols // QK_K
    size = Q2K_BYTES if kind == "q2k" else Q3K_BYTES
    blocks = np.asarray(raw, dtype=np.uint8).reshape(n_rows, nb, size)
    w = dequant_q2k(blocks) if kind == "q2k" else dequant_q3k(blocks)
    return w.reshape(n_rows, n_cols)


# ----------------------------------------------------------------------------- q8_1

def _round_half_away(v):
    v = np.asarray(v, dtype=np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def quantize_q8_1(x):
    """q8_1 of f32 values [..., K] (K % 32 == 0).

    Per 32-value block: amax = max|x|; d = amax / 127 (f32 division);
    q = round-half-away-from-zero(x / d) with the unrounded f32 d (q = 0 when
    d = 0); the stored scale is fp16(d) and the stored sum fp16(d * sum(q)).
    Returns (q int8 [..., K], d16 float64 [..., K/32], s16 float64 [..., K/32]).
    """
    x = np.asarray(x, dtype=np.float32)
    k = x.shape[-1]
    assert k % Q8_BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (k // Q8_BLOCK, Q8_BLOCK))
    amax = np.max(np.abs(xb), axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (xb / d[..., None]).astype(np.float32)
    q = np.where(d[..., None] == 0, 0.0, _round_half_away(ratio))
    q = q.astype(np.int64)
    d16 = fp16_rne(d)
    s16 = fp16_rne((d.astype(np.float32) * q.sum(axis=-1).astype(np.float32)).astype(np.float32))
    return q.reshape(x.shape).astype(np.int8), d16, s16


def q8_1_values(q, d16):
    """The values a q8_1 block stands for: fp16(d) * q, in float64."""
    q = np.asarray(q, dtype=np.int64)
    k = q.shape[-1]
    qb = q.reshape(q.shape[:-1] + (k // Q8_BLOCK, Q8_BLOCK)).astype(np.float64)
    return (qb * np.asarray(d16)[..., None]).reshape(q.shape)


# ----------------------------------------------------------------------------- MXFP4

FP4_BLOCK = 32      # weights per E8M0 scale


def e2m1_value(code):
    """e2m1 code(s) (0..15) -> float64: bit 3 the sign, bits 2-1 the exponent
    (bias 1; 0 is subnormal), bit 0 the mantissa."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    mant = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * mant, np.exp2(e - 1.0) * (1.0 + 0.5 * mant))
    return sign * mag


def e8m0_value(byte):
    """E8M0 scale byte(s) -> 2^(E - 127) as float64 (NaN for 255)."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def dequant_mxfp4(raw, n_rows, n_cols):
    """uint8 bytes of one MXFP4 matrix [codes n_rows x n_cols/2 | scales n_rows x
    n_cols/32] -> float64 [n_rows, n_cols]."""
    raw = np.asarray(raw, dtype=np.uint8).reshape(-1)
    nc = n_rows * n_cols // 2
    assert raw.size == nc + n_rows * n_cols // FP4_BLOCK, raw.size
    codes = raw[:nc].reshape(n_rows, n_cols // 2)
    lo = e2m1_value(codes & 15)
    hi = e2m1_value(codes >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(n_rows, n_cols)
    scale = e8m0_value(raw[nc:].reshape(n_rows, n_cols // FP4_BLOCK))
    return vals * np.repeat(scale, FP4_BLOCK, axis=1)
