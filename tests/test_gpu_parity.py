"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bars: routing indices bit-exact except for near-ties (gap < 1e-5 on the
oracle's keys, counted); outputs within 2e-3 * max|y| + half a bf16 ulp of the
oracle's unrounded y; q8_1 quants and scales bit-exact.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_gemv_amd as moe
import oracle
import synthetic as S
from layer_fixture import Layer, bits, compare_routing

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def check_layer(layer, x, label, sample_rows=None):
    m = x.shape[0]
    say(f"[{label}] forward m={m}")
    out, gw, idx = layer.forward(x.to(layer.dev))
    rc = layer.check()
    assert rc == moe.MOE_OK, moe.strerror(rc)
    idx_h, gw_h = idx.cpu().numpy(), gw.cpu().numpy()
    ridx, rg, rkeys, _ = layer.oracle_route(x)
    exempt = compare_routing(idx_h, gw_h, ridx, rg, rkeys)
    rows = list(range(m)) if sample_rows is None else sample_rows(idx_h) if callable(sample_rows) else sample_rows
    say(f"[{label}] routing ok ({exempt} near-tie exemptions); oracle on rows {rows}")
    # several rows of a real-shape layer: the oracle in worker processes
    ref = layer.oracle_parallel(x[rows]) if len(rows) > 2 and layer.shape.dim >= 2048 else layer.oracle(x[rows])
    got = out.float().cpu().numpy().astype(np.float64)[rows]
    worst = 0.0
    for j, t in enumerate(rows):
        if list(idx_h[t]) != list(ref["idx"][j]):
            continue   # an exempted near-tie: the two sides used different experts
        ok, ratio = oracle.within_tolerance(got[j], ref["y"][j])
        assert ok, f"{label}: token {t} off by {ratio:.3f} x tolerance"
        worst = max(worst, ratio)
    say(f"[{label}] outputs ok, worst {worst:.4f} of tolerance")
    return out, gw, idx


# ----------------------------------------------------------------------------- q8_1

def test_quantize_q8_1_bit_exact():
    torch.manual_seed(0)
    rows, cols = 37, 1024
    x = (torch.randn(rows, cols) * torch.exp2(torch.randint(-6, 6, (rows, 1)).float())).to(torch.bfloat16)
    x[0, :32] = 0                                 # zero block
    x[1, :32] = torch.tensor([127.0, 2.5, -2.5, 0.5, -0.5] + [0.0] * 27).to(torch.bfloat16)   # ties
    x[2, 32:64] = -3.0                            # constant block
    d_x = x.cuda()
    q = torch.empty(rows, cols, dtype=torch.int8, device="cuda")
    d = torch.empty(rows, cols // 32, dtype=torch.float32, device="cuda")
    moe.moe_quantize_q8_1(d_x, rows, cols, q, d)
    torch.cuda.synchronize()
    rq, rd, _ = oracle.quantize_q8_1(oracle.bf16_bits_to_f64(bits(x)).astype(np.float32))
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(d.cpu().numpy().astype(np.float64), rd)


# ----------------------------------------------------------------------------- tiny layer

TINY_VARIANTS = {
    "bf16_shared": dict(),
    "kquant_shared": dict(shared_fmt="kquant"),
    "no_shared": dict(shared_fmt="none"),
    "clamps_0.25": dict(limit=0.25),
    "no_clamps": dict(limit=0.0),
    "gate_temp_2": dict(gate_temp=2.0),
    "norm_off": dict(norm=False),
}


@pytest.mark.parametrize("variant", list(TINY_VARIANTS))
@pytest.mark.parametrize("m", [1, 4, 13, 70])
def test_tiny_layer(variant, m):
    layer = Layer(S.TINY, 0, max_tokens=80, **TINY_VARIANTS[variant])
    try:
        x = S.make_tokens(m, S.TINY.dim, 0, index=m)
        check_layer(layer, x, f"tiny {variant}")
    finally:
        layer.close()


@pytest.mark.parametrize("dispatch", ["mixed", "mmq"])
@pytest.mark.parametrize("shared", ["bf16", "kquant"])
@pytest.mark.parametrize("m", [24, 40, 150, 330])
def test_tiny_hot_expert_spans_chunks(shared, m, dispatch):
    # every token picks expert 3 first, so its group holds all m rows: one chunk of
    # the 17..32-row class (m=24), one ragged 64-row chunk (m=40), or several 64-row
    # chunks (m=150, 330); the other experts' groups fall in the smaller classes, or
    # (mixed dispatch) on the GEMV kernels when they have at most 8 rows
    mode = moe.MOE_DISPATCH_MIXED if dispatch == "mixed" else moe.MOE_DISPATCH_MMQ
    layer = Layer(S.TINY, 2, max_tokens=m, shared_fmt=shared, dispatch=mode)
    try:
        layer.bias[3] = 100.0
        layer.d_bias.copy_(layer.bias.to(layer.dev))
        check_layer(layer, S.make_tokens(m, 256, 2), f"hot expert m={m} {shared} {dispatch}")
    finally:
        layer.close()


@pytest.mark.parametrize("m", [1, 2, 5, 8])
def test_mid_decode_bf16_shared(m):
    # dim 1024, inter 512, top-4: the decode kernels at a shape between the tiny one and
    # the real one (256-thread gate/up workgroups, two K superblocks of W2 per row, the
    # bf16 shared expert's rows split over the routing launches and the down kernel)
    shape = S.LayerShape(1024, 512, 16, 4)
    layer = Layer(shape, 5, max_tokens=8)
    try:
        check_layer(layer, S.make_tokens(m, 1024, 5, index=m), f"mid bf16 shared m={m}")
    finally:
        layer.close()


@pytest.mark.parametrize("E", [16, 384, 512])
def test_router_launch_selects_interleaved_sizes(E):
    # up to 8 tokens on the decode kernels the router launch's last workgroup selects
    # (and buckets above one token, while E <= 384): its arrival counters must be back at
    # zero after every call, so calls of different sizes interleave on one context; each
    # matches the oracle the first time and repeats bit for bit. E = 512 takes the top-k
    # launch above one token.
    shape = S.LayerShape(512, 256, E, 6)
    layer = Layer(shape, 7, max_tokens=8)
    try:
        for m in (1, 3, 8):
            p = moe.moe_plan_call(layer.ctx, m, moe.MOE_SHARED_BF16)
            assert p["small_routing"] == 1 and p["expert_path"] == moe.MOE_PATH_DECODE
            assert (p["shared_rows_topk"] == 0) == (m == 1 or E <= 384), p
        first = {}
        for m in (1, 3, 8, 3, 1, 8, 1):
            x = S.make_tokens(m, shape.dim, 7, index=m)
            if m not in first:
                first[m] = bits(check_layer(layer, x, f"E={E} m={m}")[0])
            else:
                assert np.array_equal(bits(layer.forward(x.to(layer.dev))[0]), first[m]), f"E={E} m={m} repeat"
    finally:
        layer.close()


FP4_SHAPE = S.LayerShape(512, 256, 16, 3)     # dim != inter, so a transposed operand fails


@pytest.mark.parametrize("shared", ["bf16", "none"])
@pytest.mark.parametrize("m", [1, 3, 8, 13, 70])
def test_fp4_experts(shared, m):
    # MXFP4 routed experts: single-row chunks up to 8 tokens, chunks of up to 8 rows above
    layer = Layer(FP4_SHAPE, 6, max_tokens=80, shared_fmt=shared, expert_fmt="fp4")
    try:
        check_layer(layer, S.make_tokens(m, FP4_SHAPE.dim, 6, index=m), f"fp4 {shared} m={m}")
    finally:
        layer.close()


def test_fp4_hot_expert_and_clamps():
    # one expert takes every token (a 40-row group in 8-row chunks), clamps at 0.25
    layer = Layer(FP4_SHAPE, 7, max_tokens=40, expert_fmt="fp4", limit=0.25)
    try:
        layer.bias[5] = 100.0
        layer.d_bias.copy_(layer.bias.to(layer.dev))
        check_layer(layer, S.make_tokens(40, FP4_SHAPE.dim, 7), "fp4 hot expert")
    finally:
        layer.close()


def test_fp4_rejects_kquant_shared():
    with pytest.raises(moe.MoeError) as e:
        layer = Layer(FP4_SHAPE, 6, max_tokens=4, shared_fmt="kquant", expert_fmt="fp4")
        try:
            layer.forward(S.make_tokens(1, FP4_SHAPE.dim, 6).cuda())
        finally:
            layer.close()
    assert e.value.code == moe.MOE_EINVAL


@pytest.mark.parametrize("dims", [(8192, 2048), (2048, 8192)])
@pytest.mark.parametrize("m", [1, 3, 12])
def test_largest_dims(dims, m):
    # dim or inter at the 8192 limit: the decode kernels' widest workgroups (1024
    # threads), the bf16 shared rows' second round of pieces, and above 8 tokens
    # the MMQ tiles or (where the W2 tile does not fit LDS) the GEMV kernels
    shape = S.LayerShape(dims[0], dims[1], 4, 2)
    layer = Layer(shape, 8, max_tokens=12)
    try:
        check_layer(layer, S.make_tokens(m, shape.dim, 8, index=m), f"dims {dims} m={m}",
                    sample_rows=None if m <= 3 else [0, m - 1])
    finally:
        layer.close()


@pytest.mark.parametrize("m", [1, 12])
def test_fp4_largest_dim(m):
    shape = S.LayerShape(8192, 2048, 4, 2)        # an 8192-wide row: four pieces per lane
    layer = Layer(shape, 9, max_tokens=12, expert_fmt="fp4")
    try:
        check_layer(layer, S.make_tokens(m, shape.dim, 9, index=m), f"fp4 dims 8192x2048 m={m}",
                    sample_rows=None if m == 1 else [0, m - 1])
    finally:
        layer.close()


@pytest.mark.parametrize("m", [1, 5, 20])
def test_every_expert_picked(m):
    # k = E: every token picks all 8 experts (the selection is a full sort)
    layer = Layer(S.LayerShape(256, 256, 8, 8), 10, max_tokens=20)
    try:
        check_layer(layer, S.make_tokens(m, 256, 10, index=m), f"k=E m={m}")
    finally:
        layer.close()


@pytest.mark.parametrize("m", [1, 13])
def test_single_expert(m):
    layer = Layer(S.LayerShape(256, 256, 1, 1), 11, max_tokens=13)
    try:
        check_layer(layer, S.make_tokens(m, 256, 11, index=m), f"E=1 m={m}")
    finally:
        layer.close()


def test_tiny_topk1():
    shape = S.LayerShape(256, 256, 16, 1)
    layer = Layer(shape, 3, max_tokens=8)
    try:
        check_layer(layer, S.make_tokens(5, 256, 3), "tiny k=1")
    finally:
        layer.close()


def test_tiny_wide_topk_ragged():
    shape = S.LayerShape(512, 768, 40, 9)       # 9 picks, ragged groups, three K superblocks of W2
    layer = Layer(shape, 4, max_tokens=40, shared_fmt="kquant")
    try:
        check_layer(layer, S.make_tokens(37, 512, 4), "wide k=9 m=37", sample_rows=[0, 17, 36])
    finally:
        layer.close()


@pytest.mark.parametrize("m", [1, 5, 12])
def test_widest_routing_layer(m):
    # E = 1024 experts (16 keys per lane in the one-wavefront selection) and k = 64
    # picks, the configuration's limits: the m = 1 and m <= 8 routing kernels and,
    # at m = 12, the split-K router product with the per-token wavefront top-k
    shape = S.LayerShape(256, 256, 1024, 64)
    layer = Layer(shape, 12, max_tokens=12, expert_device="cuda")
    try:
        check_layer(layer, S.make_tokens(m, 256, 12, index=m), f"E=1024 k=64 m={m}",
                    sample_rows=None if m <= 5 else [0, m - 1])
    finally:
        layer.close()


@pytest.mark.parametrize("dim,E,k,m", [(1280, 1024, 64, 200), (1280, 384, 6, 9), (768, 100, 7, 77),
                                       (256, 1024, 1, 3000)])
def test_route_only_against_oracle(dim, E, k, m):
    # routing alone at shapes the layer tests do not reach: the router product split
    # over K unevenly (dim / 64 = 20 or 12 steps over up to 8 splits), every key
    # count per lane (2, 6, 16), and m = 3000, where the logits scratch leaves no room
    # for a second split. The experts are irrelevant here (zero slices).
    shape = S.LayerShape(dim, 256, E, k)
    zeros = torch.zeros((E, S.expert_layout(shape)[0]), dtype=torch.uint8, device="cuda")
    layer = Layer(shape, 13, max_tokens=m, experts=zeros, router_std=0.02)
    try:
        x = S.make_tokens(m, dim, 13).cuda()
        gw = torch.empty(m, k, dtype=torch.float32, device="cuda")
        idx = torch.empty(m, k, dtype=torch.int32, device="cuda")
        say(f"[route dim={dim} E={E} k={k} m={m}]")
        moe.moe_route(layer.ctx, layer.w, x, m, gw, idx)
        assert layer.check() == moe.MOE_OK
        ridx, rg, rkeys, _ = layer.oracle_route(x)
        exempt = compare_routing(idx.cpu().numpy(), gw.cpu().numpy(), ridx, rg, rkeys)
        say(f"[route dim={dim} E={E} k={k} m={m}] ok ({exempt} near-tie exemptions)")
    finally:
        layer.close()


def test_max_tokens():
    # m = max_tokens = 65536 (the configuration's limit): scratch sized for it, the
    # chunk lists at their bounds, routing checked for every token and the outputs on
    # sampled rows
    m = 65536
    layer = Layer(S.TINY, 14, max_tokens=m, shared_fmt="kquant")
    try:
        check_layer(layer, S.make_tokens(m, S.TINY.dim, 14), "tiny m=65536", sample_rows=[0, 12345, 40000, m - 1])
    finally:
        layer.close()


def test_tiny_deterministic():
    layer = Layer(S.TINY, 0, max_tokens=16)
    try:
        x = S.make_tokens(13, S.TINY.dim, 9).cuda()
        a = layer.forward(x)[0].clone()
        for _ in range(3):
            b = layer.forward(x)[0]
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    finally:
        layer.close()


def test_route_only_matches_forward():
    layer = Layer(S.TINY, 0, max_tokens=16)
    try:
        x = S.make_tokens(9, S.TINY.dim, 5).cuda()
        gw = torch.empty(9, 2, dtype=torch.float32, device="cuda")
        idx = torch.empty(9, 2, dtype=torch.int32, device="cuda")
        moe.moe_route(layer.ctx, layer.w, x, 9, gw, idx)
        _, gw2, idx2 = layer.forward(x)
        assert torch.equal(idx, idx2) and torch.equal(gw, gw2)
    finally:
        layer.close()


@pytest.mark.parametrize("m", [1, 2, 12])
def test_nan_key_reported(m):
    layer = Layer(S.TINY, 0, max_tokens=16)
    try:
        layer.d_bias[3] = float("nan")
        layer.forward(S.make_tokens(m, 256, 1).cuda())
        assert layer.check() == moe.MOE_ENONFINITE
        assert layer.check() == moe.MOE_OK          # the word is cleared by the read
    finally:
        layer.close()


@pytest.mark.parametrize("m", [1, 3, 12])
def test_tied_keys_pick_lowest_ids(m):
    # a zero router and zero bias: every key is sqrt(ln 2), so each token picks
    # experts 0..k-1 in that order (ties go to the lower id)
    layer = Layer(S.TINY, 0, max_tokens=16, router_std=0.0, bias=None)
    try:
        _, gw, idx = layer.forward(S.make_tokens(m, 256, 6).cuda())
        assert layer.check() == moe.MOE_OK
        k = S.TINY.topk
        assert idx.cpu().tolist() == [list(range(k))] * m
        assert torch.allclose(gw.cpu(), torch.full((m, k), 1.5 / k))
    finally:
        layer.close()


def test_not_resident_reported():
    layer = Layer(S.TINY, 0, max_tokens=4)
    try:
        x = S.make_tokens(1, 256, 2)
        ridx = layer.oracle_route(x)[0]
        moe.moe_slot_evict(layer.ctx, int(ridx[0, 0]))
        layer.forward(x.cuda())
        assert layer.check() == moe.MOE_ENOTRESIDENT
    finally:
        layer.close()


def test_invalid_arguments():
    layer = Layer(S.TINY, 0, max_tokens=4)
    try:
        x = S.make_tokens(4, 256, 2).cuda()
        out = torch.empty(5, 256, dtype=torch.bfloat16, device="cuda")
        for m in (0, 5, -1):
            with pytest.raises(moe.MoeError) as e:
                moe.moe_forward(layer.ctx, layer.w, x, m, out)
            assert e.value.code == moe.MOE_EINVAL
        with pytest.raises(moe.MoeError):
            moe.moe_slot_bind(layer.ctx, 16, 0)
        with pytest.raises(moe.MoeError):
            moe.moe_slot_bind(layer.ctx, 0, 1)          # slot 1 belongs to expert 1
    finally:
        layer.close()


# ----------------------------------------------------------------------------- real layer

@pytest.fixture(scope="module")
def real_experts():
    say("[real] drawing 384 experts on the GPU")
    a = S.make_experts(S.REAL, 1, device="cuda")
    torch.cuda.synchronize()
    yield a
    del a
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def real_fp4_experts():
    say("[real] drawing 384 MXFP4 experts on the GPU")
    a = S.make_experts(S.REAL, 1, device="cuda", fmt="fp4")
    torch.cuda.synchronize()
    yield a
    del a
    torch.cuda.empty_cache()


def test_real_fp4_decode_m1(real_fp4_experts):
    layer = Layer(S.REAL, 1, bias=(-0.05, 0.05), router_std=0.02, max_tokens=64, experts=real_fp4_experts,
                  expert_fmt="fp4")
    try:
        pool = S.make_tokens(256, S.REAL.dim, 1)
        for t in (0, 131):
            check_layer(layer, pool[t:t + 1], f"fp4 decode m=1 token {t}")
        check_layer(layer, pool[64:128], "fp4 m=64", sample_rows=[0, 63])
    finally:
        layer.close()


def test_real_decode_m1(real_experts):
    layer = Layer(S.REAL, 1, bias=(-0.05, 0.05), router_std=0.02, max_tokens=8, experts=real_experts)
    try:
        pool = S.make_tokens(256, S.REAL.dim, 1)
        for t in (0, 131):
            check_layer(layer, pool[t:t + 1], f"decode m=1 token {t}")
    finally:
        layer.close()


def test_real_decode_pool_every_token(real_experts):
    # every token of the 256-token decode pool through the one-token path (router
    # launch with its selection, gate/up, down + combine): routing against the
    # oracle for all of them, outputs for eight spread over the pool
    layer = Layer(S.REAL, 1, bias=(-0.05, 0.05), router_std=0.02, max_tokens=8, experts=real_experts)
    try:
        pool = S.make_tokens(256, S.REAL.dim, 1)
        d_pool = pool.to(layer.dev)
        outs, gws, idxs = [], [], []
        say("[decode pool] 256 one-token calls")
        for t in range(256):
            out, gw, idx = layer.forward(d_pool[t:t + 1])
            outs.append(out)
            gws.append(gw)
            idxs.append(idx)
        rc = layer.check()
        assert rc == moe.MOE_OK, moe.strerror(rc)
        idx_h = torch.cat(idxs).cpu().numpy()
        gw_h = torch.cat(gws).cpu().numpy()
        ridx, rg, rkeys, _ = layer.oracle_route(pool)
        exempt = compare_routing(idx_h, gw_h, ridx, rg, rkeys)
        say(f"[decode pool] routing of 256 tokens ok ({exempt} near-tie exemptions)")
        rows = [3, 40, 77, 111, 150, 188, 222, 255]
        ref = layer.oracle_parallel(pool[rows])
        got = torch.cat([outs[t] for t in rows]).float().cpu().numpy().astype(np.float64)
        worst = 0.0
        for j, t in enumerate(rows):
            if list(idx_h[t]) != list(ref["idx"][j]):
                continue   # an exempted near-tie
            ok, ratio = oracle.within_tolerance(got[j], ref["y"][j])
            assert ok, f"decode pool: token {t} off by {ratio:.3f} x tolerance"
            worst = max(worst, ratio)
        say(f"[decode pool] outputs of tokens {rows} ok, worst {worst:.4f} of tolerance")
    finally:
        layer.close()


def test_real_small_batch_m8_kquant_shared(real_experts):
    layer = Layer(S.REAL, 1, bias=(-0.05, 0.05), router_std=0.02, max_tokens=8, experts=real_experts,
                  shared_fmt="kquant")
    try:
        x = S.make_tokens(8, S.REAL.dim, 1, index=1)
        check_layer(layer, x, "small batch m=8")   # all eight rows
    finally:
        layer.close()


PREFILL_ROWS = [0, 31, 63, 64, 97, 128, 170, 213, 255, 256, 300, 341, 383, 384, 447, 480, 511]


@pytest.mark.parametrize("dispatch", ["mixed", "mmq"])
def test_real_prefill_m512(real_experts, dispatch):
    # uniform routing: about 8 rows per expert, so the mixed dispatch runs both the
    # GEMV kernels (groups of <= 8 rows) and the MMQ classes
    mode = moe.MOE_DISPATCH_MIXED if dispatch == "mixed" else moe.MOE_DISPATCH_MMQ
    layer = Layer(S.REAL, 1, bias=None, router_std=0.02, max_tokens=512, experts=real_experts, dispatch=mode)
    try:
        x = S.make_tokens(512, S.REAL.dim, 1, index=2)
        check_layer(layer, x, f"prefill m=512 {dispatch}", sample_rows=PREFILL_ROWS)
    finally:
        layer.close()


HOT_EXPERTS = (5, 77, 140, 203, 266, 329)
# every token picks the six hot experts, so group g holds all 512 tokens in token
# order and its 64-row chunks end at tokens 63, 127, ...: rows on both sides of
# every boundary, and the first and last rows
HOT_ROWS = [0, 1, 63, 64, 127, 128, 191, 192, 255, 256, 319, 320, 383, 384, 447, 448, 510, 511]


def test_real_prefill_hot_experts(real_experts):
    # six 512-row groups, each eight 64-row chunks over 20 superblocks of K (gate/up)
    # and 9 (down): the shape where the int8 matrix cores bind
    bias = torch.zeros(S.REAL.n_routed)
    bias[list(HOT_EXPERTS)] = 100.0
    layer = Layer(S.REAL, 1, bias=bias, router_std=0.02, max_tokens=512, experts=real_experts)
    try:
        x = S.make_tokens(512, S.REAL.dim, 1, index=2)
        _, _, idx = check_layer(layer, x, "prefill hot experts m=512", sample_rows=HOT_ROWS)
        assert sorted(set(idx.cpu().numpy().reshape(-1).tolist())) == sorted(HOT_EXPERTS)
    finally:
        layer.close()


# ----------------------------------------------------------------------------- random block bytes

def random_byte_experts(shape, seed):
    return torch.stack([S.random_kquant_slot(shape, seed + e) for e in range(shape.n_routed)])


@pytest.mark.parametrize("m", [1, 5, 8, 24, 70])
@pytest.mark.parametrize("shared", ["bf16", "kquant"])
def test_random_block_bytes(m, shared):
    # blocks no encoder writes: random scales, quants and high bits, fp16 d and dmin
    # of either sign; m <= 8 runs the decode kernels, above that the MMQ classes
    shape = S.LayerShape(512, 256, 16, 3)
    experts = random_byte_experts(shape, 40)
    layer = Layer(shape, 4, max_tokens=max(m, 8), experts=experts, shared_fmt=shared)
    try:
        if shared == "kquant":
            # the K-quant shared expert's blocks random as well
            layer.shared = {"fmt": "kquant", "slot": S.random_kquant_slot(shape, 99)}
            kcfg = moe.make_cfg(shape.dim, shape.inter, shape.n_routed, shape.topk, max_tokens=max(m, 8))
            moe.moe_pack_expert(kcfg, layer.shared["slot"].cuda(), layer.d_shared["slot"])
        check_layer(layer, S.make_tokens(m, shape.dim, 4, index=m), f"random bytes m={m} {shared}")
    finally:
        layer.close()


@pytest.mark.parametrize("m", [40, 150])
def test_random_block_bytes_hot_expert(m):
    # one expert takes every token: multi-chunk MMQ groups over random blocks
    shape = S.LayerShape(512, 256, 16, 2)
    bias = torch.zeros(16)
    bias[9] = 100.0
    layer = Layer(shape, 6, max_tokens=m, experts=random_byte_experts(shape, 60), bias=bias)
    try:
        check_layer(layer, S.make_tokens(m, shape.dim, 6, index=m), f"random bytes hot m={m}")
    finally:
        layer.close()


# ----------------------------------------------------------------------------- counters

@pytest.mark.parametrize("m", [1, 3, 12])
def test_near_ties_counted(m):
    # a zero router: every score is sqrt(ln 2), so the keys follow the bias; expert 1
    # (the 2nd pick) lies 4e-6 above expert 2, a near tie at the k / k+1 boundary
    bias = torch.zeros(16)
    bias[0], bias[1], bias[2] = 0.5, 0.3 + 4e-6, 0.3
    layer = Layer(S.TINY, 0, max_tokens=16, router_std=0.0, bias=bias)
    try:
        x = S.make_tokens(m, 256, 6).cuda()
        moe.moe_reset_stats(layer.ctx)
        _, _, idx = layer.forward(x)
        assert layer.check() == moe.MOE_OK
        assert idx.cpu().tolist() == [[0, 1]] * m
        st = moe.moe_get_stats(layer.ctx)
        assert st["near_ties"] == m and st["calls"] == 1
        gw = torch.empty(m, 2, device="cuda")
        moe.moe_route(layer.ctx, layer.w, x, m, gw, idx)
        assert moe.moe_get_stats(layer.ctx)["near_ties"] == 2 * m
        moe.moe_reset_stats(layer.ctx)
        assert moe.moe_get_stats(layer.ctx)["near_ties"] == 0
        # a clear gap: none
        layer.d_bias[1] = 0.4
        layer.forward(x)
        assert moe.moe_get_stats(layer.ctx)["near_ties"] == 0
    finally:
        layer.close()


def test_compute_time_with_profiling():
    layer = Layer(S.TINY, 0, max_tokens=16)
    try:
        x = S.make_tokens(12, 256, 1).cuda()
        moe.moe_reset_stats(layer.ctx)
        layer.forward(x)
        assert moe.moe_get_stats(layer.ctx)["compute_ms"] == 0.0    # no events without profiling
        moe.moe_set_profiling(layer.ctx, True)
        for m in (1, 12):
            layer.forward(x[:m])
        st = moe.moe_get_stats(layer.ctx)
        moe.moe_set_profiling(layer.ctx, False)
        assert st["compute_ms"] > 0 and st["calls"] == 3
    finally:
        layer.close()


# ----------------------------------------------------------------------------- drawn configurations

def drawn_configs(n, seed):
    """n layer configurations drawn from the ones the library accepts (dims multiples
    of 256, any expert count, top-k up to min(E, 64)), small enough for the oracle,
    each with a token count on one of the paths (1, 2..8, above 8)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dim = 256 * int(rng.integers(1, 5))
        inter = 256 * int(rng.integers(1, 5))
        E = int(rng.choice([3, 8, 17, 37, 64, 100, 129, 200, 385]))
        k = int(rng.integers(1, min(E, 9) + 1))
        m = int(rng.choice([1, 2, 5, 8, 9, 20, 47]))
        shared = str(rng.choice(["bf16", "kquant", "none"]))
        out.append((dim, inter, E, k, m, shared))
    return out


@pytest.mark.parametrize("dim,inter,E,k,m,shared", drawn_configs(16, 2024))
def test_drawn_configuration(dim, inter, E, k, m, shared):
    layer = Layer(S.LayerShape(dim, inter, E, k), 7, max_tokens=m, shared_fmt=shared)
    try:
        x = S.make_tokens(m, dim, 7, index=E + k)
        check_layer(layer, x, f"drawn {dim}x{inter} E={E} k={k} m={m} {shared}")
    finally:
        layer.close()


@pytest.mark.parametrize("dim,inter,E,k,m,shared", [(d, i, e, k, m, "none" if s == "kquant" else s)
                                                     for d, i, e, k, m, s in drawn_configs(8, 77)])
def test_drawn_configuration_fp4(dim, inter, E, k, m, shared):
    layer = Layer(S.LayerShape(dim, inter, E, k), 8, max_tokens=m, shared_fmt=shared, expert_fmt="fp4")
    try:
        x = S.make_tokens(m, dim, 8, index=E + k)
        check_layer(layer, x, f"drawn fp4 {dim}x{inter} E={E} k={k} m={m} {shared}")
    finally:
        layer.close()
