"""Seeded generators for the MoE layer's inputs (torch; CPU or GPU).

Recipe (shapes and distributions of the pages' layer, DeepSeek-V4.1 config:
dim 5120, moe_inter_dim 2304, 384 routed experts, 6 active, 1 shared):
  * router weight bf16 [n_routed, dim] ~ N(0, std_router) rounded to bf16 (RNE);
  * bias f32 [n_routed] ~ U(lo, hi), or zero, or the skewed ranking below;
  * routed expert e: W1, W3 [inter, dim] and W2 [dim, inter] drawn f32 ~ N(0, 0.02)
    and packed into Q2_K (W1, W3) and Q3_K (W2) blocks; the expert's slice is
    [W1 | W3 | W2] raw block bytes, rows in order; or (fmt "fp4") the same draws
    packed as microscaled FP4: per 32 weights of a row one E8M0 power-of-two
    scale and 32 e2m1 codes, each matrix [codes rows x cols/2 | scales rows x cols/32];
  * shared expert: the same draws kept as bf16, or packed like a routed expert;
  * tokens bf16 [m, dim] ~ N(0, 1) rounded to bf16.
Every stream has its own seed derived from (seed, tag, index, matrix), so any
expert can be regenerated alone. Router, bias, shared expert and tokens are
always drawn on the CPU (identical on every machine); the 4.9 GB of routed
blocks may be drawn on the GPU, where the stream differs from the CPU one, so a
check against the oracle copies the blocks it needs back from the device.
"""

from dataclasses import dataclass

import numpy as np
import torch

QK = 256
Q2K_BYTES = 84
Q3K_BYTES = 110

TAG_ROUTER, TAG_BIAS, TAG_EXPERT, TAG_SHARED, TAG_TOKENS, TAG_PERM = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class LayerShape:
    dim: int
    inter: int
    n_routed: int
    topk: int


TINY = LayerShape(dim=256, inter=256, n_routed=16, topk=2)
REAL = LayerShape(dim=5120, inter=2304, n_routed=384, topk=6)

# Scale c of the skewed bias b_e = -c * 1.1 * ln(rank_e) (mean removed) for the
# 2048-token skewed prefill on the real layer (seed 1). Calibrated so the 38 most
# loaded experts take 50 +- 1 % of the assignments; tests/golden/make_c4_bias.py
# wrote it and tests/test_synthetic.py checks it with the oracle's router.
C4_BIAS_SCALE = 0.143256


def stream_seed(seed, tag, index=0, matrix=0):
    """A 63-bit seed for one named stream."""
    ss = np.random.SeedSequence([int(seed), int(tag), int(index), int(matrix)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def f32_normal(shape, std, seed, device="cpu"):
    g = _gen(seed, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def bf16_normal(shape, std, seed, device="cpu"):
    """N(0, std) draws rounded to bf16 (round to nearest even)."""
    return f32_normal(shape, std, seed, device).to(torch.bfloat16)


def uniform_f32(shape, lo, hi, seed, device="cpu"):
    g = _gen(seed, device)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def _fp16_bytes(v):
    """float tensor [n] -> uint8 [n, 2] little-endian binary16."""
    return v.to(torch.float16).contiguous().view(torch.uint8).reshape(-1, 2)


def encode_q2k(w):
    """f32 [rows, cols] (cols % 256 == 0) -> Q2_K blocks uint8 [rows, cols/256*84].

    Min/max encoder per 16-weight sub-block: lo = min(0, min w), step = (max w - lo)/3,
    sub-block scale and min as 4-bit multiples of the superblock's fp16 d and dmin.
    """
    rows, cols = w.shape
    nb = rows * cols // QK
    x = w.reshape(nb, 16, 16).float()
    lo = torch.clamp(x.amin(-1), max=0.0)
    hi = x.amax(-1)
    step = (hi - lo) / 3.0
    mn = -lo
    d = (step.amax(-1) / 15.0).to(torch.float16).float()
    dmin = (mn.amax(-1) / 15.0).to(torch.float16).float()
    sc = torch.where(d[:, None] > 0, torch.round(step / d[:, None].clamp_min(1e-30)), torch.zeros_like(step))
    sc = sc.clamp(0, 15)
    m = torch.where(dmin[:, None] > 0, torch.round(mn / dmin[:, None].clamp_min(1e-30)), torch.zeros_like(mn))
    m = m.clamp(0, 15)
    unit = (d[:, None] * sc)[..., None]
    off = (dmin[:, None] * m)[..., None]
    q = torch.where(unit > 0, torch.round((x + off) / unit.clamp_min(1e-30)), torch.zeros_like(x))
    q = q.clamp(0, 3).to(torch.int32).reshape(nb, 2, 4, 32)  # [block, half h, plane j, position l]
    qs = torch.zeros(nb, 2, 32, dtype=torch.int32, device=w.device)
    for j in range(4):
        qs |= q[:, :, j, :] << (2 * j)
    scales = (sc.to(torch.int32) | (m.to(torch.int32) << 4)).to(torch.uint8)
    out = torch.cat(
        [scales, qs.reshape(nb, 64).to(torch.uint8), _fp16_bytes(d), _fp16_bytes(dmin)], dim=1
    )
    return out.reshape(rows, (cols // QK) * Q2K_BYTES)


def encode_q3k(w):
    """f32 [rows, cols] -> Q3_K blocks uint8 [rows, cols/256*110].

    Per 16-weight sub-block the signed value of largest magnitude maps to q3 = -4;
    the sub-block scales are 6-bit signed multiples of the superblock's fp16 d.
    """
    rows, cols = w.shape
    nb = rows * cols // QK
    x = w.reshape(nb, 16, 16).float()
    pos = x.abs().argmax(-1, keepdim=True)
    vmax = torch.gather(x, -1, pos)[..., 0]
    scale = vmax / -4.0
    d = (scale.abs().amax(-1) / 32.0).to(torch.float16).float()
    s = torch.where(d[:, None] > 0, torch.round(scale / d[:, None].clamp_min(1e-30)), torch.zeros_like(scale))
    s = s.clamp(-32, 31)
    unit = (d[:, None] * s)[..., None]
    q3 = torch.where(unit != 0, torch.round(x / torch.where(unit != 0, unit, torch.ones_like(unit))), torch.zeros_like(x))
    q3 = q3.clamp(-4, 3).to(torch.int32) + 4          # 0..7 = low 2 bits + 4 * high bit
    q3 = q3.reshape(nb, 2, 4, 32)                      # [block, h, j, l]
    low = q3 & 3
    high = q3 >> 2
    qs = torch.zeros(nb, 2, 32, dtype=torch.int32, device=w.device)
    hmask = torch.zeros(nb, 32, dtype=torch.int32, device=w.device)
    for h in range(2):
        for j in range(4):
            qs[:, h, :] |= low[:, h, j, :] << (2 * j)
            hmask |= high[:, h, j, :] << (4 * h + j)
    sc6 = (s + 32).to(torch.int32)                     # [nb, 16], 0..63
    low4 = sc6 & 15
    hi2 = sc6 >> 4
    b0_7 = low4[:, 0:8] | (low4[:, 8:16] << 4)
    b8_11 = torch.zeros(nb, 4, dtype=torch.int32, device=w.device)
    for quarter in range(4):
        b8_11 |= hi2[:, 4 * quarter:4 * quarter + 4] << (2 * quarter)
    out = torch.cat(
        [
            hmask.to(torch.uint8),
            qs.reshape(nb, 64).to(torch.uint8),
            b0_7.to(torch.uint8),
            b8_11.to(torch.uint8),
            _fp16_bytes(d),
        ],
        dim=1,
    )
    return out.reshape(rows, (cols // QK) * Q3K_BYTES)


FP4_BLOCK = 32                                    # weights per E8M0 scale
_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)   # between the magnitudes 0 .5 1 1.5 2 3 4 6


def encode_mxfp4(w):
    """f32 [rows, cols] (cols % 32 == 0) -> uint8 [rows * cols/2 + rows * cols/32]:
    the codes [rows, cols/2] (weight 2i of a row in the low nibble of byte i, 2i + 1
    in the high nibble), then the scales [rows, cols/32].

    Per 32-weight block: E = 127 + ceil(log2(amax / 6)) (clamped to 1..254; 127 for
    an all-zero block), so |w| / 2^(E-127) <= 6; each weight is coded as the sign
    bit (bit 3) and the index (bits 0-2) of the nearest e2m1 magnitude.
    """
    rows, cols = w.shape
    x = w.reshape(rows, cols // FP4_BLOCK, FP4_BLOCK).float()
    amax = x.abs().amax(-1)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax.clamp_min(1e-38) / 6.0)), torch.zeros_like(amax))
    e = (e + 127).clamp(1, 254)
    scale = torch.exp2(e - 127)[..., None]
    mag = (x.abs() / scale).clamp(max=6.0)
    mids = torch.tensor(_E2M1_MIDPOINTS, dtype=torch.float32, device=w.device)
    idx = torch.bucketize(mag, mids).to(torch.int32)            # 0..7
    code = idx | torch.where((x < 0) & (idx > 0), 8, 0).to(torch.int32)
    code = code.reshape(rows, cols // 2, 2)
    packed = (code[..., 0] | (code[..., 1] << 4)).to(torch.uint8)
    return torch.cat([packed.reshape(-1), e.to(torch.uint8).reshape(-1)])


def mxfp4_bytes(rows, cols):
    return rows * cols // 2 + rows * cols // FP4_BLOCK


def expert_layout(shape, fmt="kquant"):
    """(slot_bytes, off_w1, off_w3, off_w2) of one expert slice [W1 | W3 | W2]."""
    if fmt == "fp4":
        n13 = mxfp4_bytes(shape.inter, shape.dim)
        n2 = mxfp4_bytes(shape.dim, shape.inter)
    else:
        n13 = shape.inter * (shape.dim // QK) * Q2K_BYTES
        n2 = shape.dim * (shape.inter // QK) * Q3K_BYTES
    return 2 * n13 + n2, 0, n13, 2 * n13


def _slot_from_f32(shape, w1, w3, w2, out=None, fmt="kquant"):
    size, o1, o3, o2 = expert_layout(shape, fmt)
    if out is None:
        out = torch.empty(size, dtype=torch.uint8, device=w1.device)
    if fmt == "fp4":
        out[o1:o3] = encode_mxfp4(w1)
        out[o3:o2] = encode_mxfp4(w3)
        out[o2:] = encode_mxfp4(w2)
    else:
        out[o1:o3] = encode_q2k(w1).reshape(-1)
        out[o3:o2] = encode_q2k(w3).reshape(-1)
        out[o2:] = encode_q3k(w2).reshape(-1)
    return out


def make_expert_slot(shape, seed, expert, std=0.02, device="cpu", out=None, fmt="kquant"):
    """Routed expert `expert`'s slice as uint8 [slot_bytes] on `device`."""
    w1 = f32_normal((shape.inter, shape.dim), std, stream_seed(seed, TAG_EXPERT, expert, 0), device)
    w3 = f32_normal((shape.inter, shape.dim), std, stream_seed(seed, TAG_EXPERT, expert, 1), device)
    w2 = f32_normal((shape.dim, shape.inter), std, stream_seed(seed, TAG_EXPERT, expert, 2), device)
    return _slot_from_f32(shape, w1, w3, w2, out, fmt)


def make_experts(shape, seed, std=0.02, device="cpu", experts=None, fmt="kquant"):
    """All routed experts as one uint8 arena [n_routed, slot_bytes] (row e = expert e)."""
    size = expert_layout(shape, fmt)[0]
    n = shape.n_routed
    arena = torch.empty((n, size), dtype=torch.uint8, device=device)
    for e in range(n) if experts is None else experts:
        make_expert_slot(shape, seed, e, std, device, out=arena[e], fmt=fmt)
    return arena


def random_kquant_slot(shape, seed, d_log2=(-10.0, -8.0), d3_log2=(-12.0, -10.0)):
    """An expert slice [W1 | W3 | W2] of random block bytes: every scale nibble,
    six-bit scale, quant and hmask bit drawn uniformly, and the fp16 d (and
    dmin) fields replaced by finite values of random sign with |d| = 2^u, u
    uniform in d_log2 (Q2_K d and dmin) or d3_log2 (Q3_K d), so the weights stay
    finite and of moderate size. Blocks no min/max encoder would write."""
    size, o1, o3, o2 = expert_layout(shape)
    g = _gen(stream_seed(seed, TAG_EXPERT, 1 << 20), "cpu")
    raw = torch.randint(0, 256, (size,), generator=g, dtype=torch.int32).to(torch.uint8)

    def fp16_fields(n, lo_hi):
        mag = torch.exp2(torch.rand(n, generator=g) * (lo_hi[1] - lo_hi[0]) + lo_hi[0])
        sign = torch.where(torch.rand(n, generator=g) < 0.5, -1.0, 1.0)
        return _fp16_bytes(mag * sign)

    n13 = shape.inter * (shape.dim // QK)
    for off in (o1, o3):
        blocks = raw[off:off + n13 * Q2K_BYTES].view(n13, Q2K_BYTES)
        blocks[:, 80:82] = fp16_fields(n13, d_log2)
        blocks[:, 82:84] = fp16_fields(n13, d_log2)
    n2 = shape.dim * (shape.inter // QK)
    blocks = raw[o2:o2 + n2 * Q3K_BYTES].view(n2, Q3K_BYTES)
    blocks[:, 108:110] = fp16_fields(n2, d3_log2)
    return raw


def make_router(shape, seed, std, bias=(-0.1, 0.1)):
    """(router bf16 [n_routed, dim], bias f32 [n_routed]) on the CPU.
    bias: (lo, hi) for U(lo, hi), None for zero, or a tensor."""
    wr = bf16_normal((shape.n_routed, shape.dim), std, stream_seed(seed, TAG_ROUTER))
    if bias is None:
        b = torch.zeros(shape.n_routed, dtype=torch.float32)
    elif isinstance(bias, torch.Tensor):
        b = bias.to(torch.float32)
    else:
        b = uniform_f32((shape.n_routed,), bias[0], bias[1], stream_seed(seed, TAG_BIAS))
    return wr, b


def make_shared(shape, seed, fmt, std=0.02):
    """Shared expert on the CPU: {"fmt": "bf16", w1, w3, w2 bf16} or
    {"fmt": "kquant", "slot": uint8 [slot_bytes]}, both from the same f32 draws."""
    w1 = f32_normal((shape.inter, shape.dim), std, stream_seed(seed, TAG_SHARED, 0, 0))
    w3 = f32_normal((shape.inter, shape.dim), std, stream_seed(seed, TAG_SHARED, 0, 1))
    w2 = f32_normal((shape.dim, shape.inter), std, stream_seed(seed, TAG_SHARED, 0, 2))
    if fmt == "bf16":
        return {"fmt": "bf16", "w1": w1.to(torch.bfloat16), "w3": w3.to(torch.bfloat16),
                "w2": w2.to(torch.bfloat16)}
    if fmt == "kquant":
        return {"fmt": "kquant", "slot": _slot_from_f32(shape, w1, w3, w2)}
    raise ValueError(fmt)


def make_tokens(m, dim, seed, index=0, std=1.0):
    """bf16 [m, dim] ~ N(0, std) on the CPU; `index` selects an independent batch."""
    return bf16_normal((m, dim), std, stream_seed(seed, TAG_TOKENS, index))


def skewed_bias(shape, seed, c):
    """b_e = -c * 1.1 * ln(rank_e), rank a seeded permutation of 1..n, mean removed."""
    g = _gen(stream_seed(seed, TAG_PERM), "cpu")
    rank = torch.randperm(shape.n_routed, generator=g).to(torch.float64) + 1.0
    b = -c * 1.1 * torch.log(rank)
    return (b - b.mean()).to(torch.float32)
