"""GPU: the decode step captured in a HIP graph replays bit for bit like the
eager call (the pages' compute_m1: no per-token host arguments, so one graph
of it replays for any token written into its input buffer); likewise small
batches (the router launch's selection and bucketing) and a batched call (the
split-K router product, top-k, bucketing, MMQ classes and a bf16 shared expert
forked to a second stream inside the capture).

Every replay is checked against an eager call of the same token, with the
eager work and a synchronisation between replays.
"""
import pytest
import torch

import mixture_experts_ffn_gemv_amd as moe
import synthetic as S
from layer_fixture import Layer
from test_gpu_parity import real_experts  # noqa: F401 (module fixture)

pytestmark = pytest.mark.gpu


def capture_and_compare(layer, tokens, label, m=1):
    dev = layer.dev
    x_static = torch.zeros((m, layer.shape.dim), dtype=torch.bfloat16, device=dev)
    out_static = torch.empty((m, layer.shape.dim), dtype=torch.bfloat16, device=dev)
    x_static.copy_(tokens[0:m].to(dev))
    moe.moe_forward(layer.ctx, layer.w, x_static, m, out_static)   # uploads the slot table before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_forward(layer.ctx, layer.w, x_static, m, out_static)
    torch.cuda.synchronize()
    for t in range(tokens.shape[0] // m):
        x = tokens[t * m:(t + 1) * m].to(dev)
        x_static.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        got = out_static.clone()
        ref = torch.empty_like(out_static)
        moe.moe_forward(layer.ctx, layer.w, x, m, ref)   # eager work between replays
        torch.cuda.synchronize()
        assert layer.check() == moe.MOE_OK
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{label}: token {t} differs"
    print(f"[{label}] {tokens.shape[0] // m} replays bit-identical to eager", flush=True)


@pytest.mark.parametrize("shared", ["bf16", "kquant", "none"])
def test_tiny_decode_graph(shared):
    layer = Layer(S.TINY, 0, max_tokens=8, shared_fmt=shared)
    try:
        capture_and_compare(layer, S.make_tokens(6, S.TINY.dim, 0, index=50), f"tiny graph {shared}")
    finally:
        layer.close()


@pytest.mark.parametrize("shared", ["bf16", "kquant"])
@pytest.mark.parametrize("m", [3, 8, 13])
def test_tiny_batch_graph(shared, m):
    # m = 3 and 8: the small-batch path (selection and bucketing in the router launch);
    # m = 13: router GEMM split over K, top-k, bucketing, MMQ (bf16 shared: a second stream)
    layer = Layer(S.TINY, 0, max_tokens=16, shared_fmt=shared)
    try:
        capture_and_compare(layer, S.make_tokens(4 * m, S.TINY.dim, 0, index=70 + m), f"tiny graph m={m} {shared}", m=m)
    finally:
        layer.close()


@pytest.mark.parametrize("shared", ["bf16", "none"])
def test_tiny_fp4_decode_graph(shared):
    layer = Layer(S.LayerShape(512, 256, 16, 3), 2, max_tokens=8, shared_fmt=shared, expert_fmt="fp4")
    try:
        capture_and_compare(layer, S.make_tokens(5, 512, 2, index=60), f"tiny fp4 graph {shared}")
    finally:
        layer.close()


def test_real_decode_graph(real_experts):
    layer = Layer(S.REAL, 1, bias=(-0.05, 0.05), router_std=0.02, max_tokens=8, experts=real_experts)
    try:
        capture_and_compare(layer, S.make_tokens(4, S.REAL.dim, 1, index=0), "real decode graph")
    finally:
        layer.close()


@pytest.mark.parametrize("dim,inter,E,k,m,shared", [c for c in __import__("test_gpu_parity").drawn_configs(6, 4242)])
def test_drawn_graph(dim, inter, E, k, m, shared):
    layer = Layer(S.LayerShape(dim, inter, E, k), 3, max_tokens=m, shared_fmt=shared)
    try:
        capture_and_compare(layer, S.make_tokens(3 * m, dim, 3, index=400 + m),
                            f"drawn graph {dim}x{inter} E={E} k={k} m={m} {shared}", m=m)
    finally:
        layer.close()
