"""GPU: moe_forward_static, the decode path with no context and no allocation
(its scratch a static device array), against moe_forward_ex of a context on
the same layer and inputs, through the C ABI.

The two run the same kernels in the same order, so outputs, weights and picks
must agree bit for bit; the static call's outputs are also held to the
oracle's bar. Each case makes two calls in a row, the second with fewer
tokens, so the second runs on the scratch the first one left behind.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_gemv_amd as moe
import oracle
import synthetic as S
from layer_fixture import Layer

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def static_call(layer, x, m, status=None):
    k = layer.shape.topk
    out = torch.empty((m, layer.shape.dim), dtype=torch.bfloat16, device="cuda")
    gw = torch.empty((m, k), dtype=torch.float32, device="cuda")
    idx = torch.empty((m, k), dtype=torch.int32, device="cuda")
    table = torch.arange(layer.shape.n_routed, dtype=torch.int32, device="cuda")
    moe.moe_forward_static(layer.cfg, layer.w, layer.arena, table, x, m, out, gw, idx, status)
    torch.cuda.synchronize()
    return out, gw, idx


def check_pair(layer, x, label, oracle_rows=True):
    m = x.shape[0]
    d_x = x.cuda()
    status = torch.zeros(2, dtype=torch.int32, device="cuda")
    say(f"[{label}] static m={m}")
    out_s, gw_s, idx_s = static_call(layer, d_x, m, status)
    say(f"[{label}] context m={m}")
    out_c, gw_c, idx_c = layer.forward(d_x)
    assert layer.check() == moe.MOE_OK
    assert status.cpu().tolist()[0] == 0
    assert torch.equal(idx_s, idx_c) and torch.equal(gw_s, gw_c)
    assert torch.equal(out_s.view(torch.int16), out_c.view(torch.int16)), f"{label}: outputs differ"
    if oracle_rows:
        ref = layer.oracle(x)
        assert np.array_equal(idx_s.cpu().numpy(), ref["idx"])
        ok, ratio = oracle.within_tolerance(out_s.float().cpu().numpy().astype(np.float64), ref["y"])
        assert ok, f"{label}: {ratio:.3f} x tolerance"
        say(f"[{label}] ok, worst {ratio:.3f} of tolerance")


@pytest.mark.parametrize("shared", ["bf16", "kquant", "none"])
def test_static_matches_context_tiny(shared):
    layer = Layer(S.TINY, 0, max_tokens=8, shared_fmt=shared)
    try:
        check_pair(layer, S.make_tokens(8, 256, 3), f"tiny {shared} first")
        check_pair(layer, S.make_tokens(3, 256, 4), f"tiny {shared} second, smaller")
    finally:
        layer.close()


def test_static_matches_context_mid():
    shape = S.LayerShape(1024, 512, 64, 6)
    layer = Layer(shape, 2, max_tokens=8)
    try:
        check_pair(layer, S.make_tokens(7, shape.dim, 2), "mid first")
        check_pair(layer, S.make_tokens(1, shape.dim, 5), "mid second, smaller")
    finally:
        layer.close()


def test_static_matches_context_real():
    experts = S.make_experts(S.REAL, 1, device="cuda")
    layer = Layer(S.REAL, 1, bias=(-0.05, 0.05), router_std=0.02, max_tokens=8, experts=experts)
    try:
        pool = S.make_tokens(16, S.REAL.dim, 1)
        check_pair(layer, pool[:8], "real first", oracle_rows=False)
        check_pair(layer, pool[8:9], "real second, one token")
    finally:
        layer.close()
        del experts
        torch.cuda.empty_cache()


def drawn_decode_configs(n, seed):
    """layer configurations drawn from the accepted range, each with two token
    counts of the decode path (m <= 8), the second smaller"""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dim = 256 * int(rng.integers(1, 5))
        inter = 256 * int(rng.integers(1, 5))
        E = int(rng.choice([3, 8, 17, 37, 64, 100, 129, 200, 385]))
        k = int(rng.integers(1, min(E, 9) + 1))
        m1 = int(rng.integers(2, 9))
        m2 = int(rng.integers(1, m1))
        shared = str(rng.choice(["bf16", "kquant", "none"]))
        out.append((dim, inter, E, k, m1, m2, shared))
    return out


@pytest.mark.parametrize("dim,inter,E,k,m1,m2,shared", drawn_decode_configs(8, 31))
def test_static_matches_context_drawn(dim, inter, E, k, m1, m2, shared):
    shape = S.LayerShape(dim, inter, E, k)
    layer = Layer(shape, 6, max_tokens=8, shared_fmt=shared)
    try:
        check_pair(layer, S.make_tokens(m1, dim, 6, index=E), f"drawn {dim}x{inter} E={E} k={k} {shared} first")
        check_pair(layer, S.make_tokens(m2, dim, 6, index=E + 1), f"drawn {dim}x{inter} E={E} k={k} second")
    finally:
        layer.close()


def test_static_status_words():
    layer = Layer(S.TINY, 0, max_tokens=8)
    try:
        x = S.make_tokens(2, 256, 7).cuda()
        status = torch.zeros(2, dtype=torch.int32, device="cuda")
        # a picked expert that is not resident: flag 2
        ridx = layer.oracle_route(x.cpu())[0]
        table = torch.arange(16, dtype=torch.int32, device="cuda")
        table[int(ridx[0, 0])] = -1
        out = torch.empty((2, 256), dtype=torch.bfloat16, device="cuda")
        moe.moe_forward_static(layer.cfg, layer.w, layer.arena, table, x, 2, out, None, None, status)
        torch.cuda.synchronize()
        assert status.cpu().tolist()[0] == 2
        # a NaN key: flag 1
        status.zero_()
        layer.d_bias[5] = float("nan")
        static_call(layer, x, 2, status)
        assert status.cpu().tolist()[0] & 1
    finally:
        layer.close()


def test_static_rejects_what_it_cannot_run():
    layer = Layer(S.TINY, 0, max_tokens=16)
    try:
        x = S.make_tokens(9, 256, 1).cuda()
        out = torch.empty((9, 256), dtype=torch.bfloat16, device="cuda")
        table = torch.arange(16, dtype=torch.int32, device="cuda")
        for m in (0, 9):
            with pytest.raises(moe.MoeError) as e:
                moe.moe_forward_static(layer.cfg, layer.w, layer.arena, table, x, m, out)
            assert e.value.code == moe.MOE_EINVAL
        fp4 = moe.make_cfg(256, 256, 16, 2, expert_fmt=moe.MOE_EXPERT_MXFP4)
        with pytest.raises(moe.MoeError) as e:
            moe.moe_forward_static(fp4, layer.w, layer.arena, table, x, 1, out)
        assert e.value.code == moe.MOE_EINVAL
    finally:
        layer.close()
