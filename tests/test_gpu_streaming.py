"""GPU: expert slots with misses streamed from a page-locked host arena.

The layer keeps fewer device slots than experts; every call reads its picks
back, copies the missing experts' slices into least-recently-used slots, and
(when the picked experts outnumber the slots) runs the expert kernels in
waves. Outputs are held to the same bar as the resident tests.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_gemv_amd as moe
import synthetic as S
from layer_fixture import Layer
from test_gpu_parity import check_layer, real_experts  # noqa: F401 (module fixture)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n_slots,shared", [
    (4, 8, "bf16"),        # small-batch path, one wave
    (8, 4, "kquant"),      # small-batch path, several waves (general kernels)
    (40, 16, "bf16"),      # MMQ path, one wave, every expert fits
    (40, 4, "bf16"),       # MMQ path, waves of two experts
    (24, 6, "kquant"),     # MMQ path, waves of three, K-quant shared expert
])
def test_streamed_layer(m, n_slots, shared):
    layer = Layer(S.TINY, 0, max_tokens=max(m, 8), shared_fmt=shared, n_slots=n_slots, bind_all=False,
                  host_arena=True)
    try:
        x = S.make_tokens(m, S.TINY.dim, 0, index=100 + m)
        moe.moe_reset_stats(layer.ctx)
        check_layer(layer, x, f"streamed m={m} slots={n_slots} {shared}")
        st = moe.moe_get_stats(layer.ctx)
        ridx = layer.oracle_route(x)[0]
        distinct = len(set(ridx.reshape(-1).tolist()))
        print(f"stats {st} distinct {distinct}", flush=True)
        assert st["hits"] + st["misses"] >= distinct
        assert st["misses"] >= distinct - min(distinct, n_slots)   # at least what could not have been resident
        assert st["bytes_copied"] == st["misses"] * layer.arena_src.shape[1]
        expect_waves = 1 if distinct <= n_slots else -(-distinct // max(1, n_slots // 2))
        assert st["waves"] == expect_waves
        # the same tokens again: with enough slots every expert is now a hit
        moe.moe_reset_stats(layer.ctx)
        out2, _, _ = layer.forward(x.cuda())
        assert layer.check() == moe.MOE_OK
        st2 = moe.moe_get_stats(layer.ctx)
        if distinct <= n_slots:
            assert st2["misses"] == 0 and st2["hits"] == distinct
        check_layer(layer, x, f"streamed again m={m} slots={n_slots}")
    finally:
        layer.close()


FP4_SHAPE = S.LayerShape(512, 256, 16, 3)


@pytest.mark.parametrize("m,n_slots", [
    (4, 8),      # small-batch path, one wave
    (8, 4),      # small-batch path, several waves
    (40, 4),     # MMQ path, waves
])
def test_streamed_fp4_layer(m, n_slots):
    # MXFP4 experts streamed in their tiled slot layout from the host arena
    layer = Layer(FP4_SHAPE, 5, max_tokens=max(m, 8), n_slots=n_slots, bind_all=False, host_arena=True,
                  expert_fmt="fp4")
    try:
        x = S.make_tokens(m, FP4_SHAPE.dim, 5, index=200 + m)
        moe.moe_reset_stats(layer.ctx)
        check_layer(layer, x, f"streamed fp4 m={m} slots={n_slots}")
        st = moe.moe_get_stats(layer.ctx)
        distinct = len(set(layer.oracle_route(x)[0].reshape(-1).tolist()))
        assert st["misses"] >= distinct - min(distinct, n_slots)
        assert st["bytes_copied"] == st["misses"] * layer.arena_src.shape[1]
        assert st["waves"] == (1 if distinct <= n_slots else -(-distinct // max(1, n_slots // 2)))
    finally:
        layer.close()


def test_streamed_lru_keeps_recent():
    # two batches that each fit the slots: the second one evicts only experts the
    # first one no longer needs, and a third call with the first batch's tokens
    # finds what is left of them
    layer = Layer(S.TINY, 1, max_tokens=8, n_slots=8, bind_all=False, host_arena=True)
    try:
        xa = S.make_tokens(2, S.TINY.dim, 1, index=7)
        xb = S.make_tokens(2, S.TINY.dim, 1, index=8)
        for x in (xa, xb, xa):
            check_layer(layer, x, "lru")
        st = moe.moe_get_stats(layer.ctx)
        assert st["calls"] == 3 and st["misses"] > 0 and st["hits"] > 0
        resident = [moe.moe_slot_of(layer.ctx, e) for e in range(S.TINY.n_routed)]
        slots = [s for s in resident if s >= 0]
        assert len(slots) == len(set(slots)) and len(slots) <= 8
    finally:
        layer.close()


def chunk_boundary_rows(idx):
    """Rows that meet every group of more than 64 rows (the groups cut into
    several 64-row chunks) on both sides of a chunk boundary: for each such
    group, largest first, not yet met by a chosen row, the tokens at positions
    63 and 64 of the group (its rows are in token order); and positions 127/128
    of the three largest groups."""
    m = idx.shape[0]
    cnt = np.bincount(idx.reshape(-1), minlength=S.REAL.n_routed)
    multi = [int(e) for e in np.argsort(-cnt, kind="stable") if cnt[e] > 64]
    members = {e: [t for t in range(m) if e in idx[t]] for e in multi}
    rows, met = set(), set()
    for e in multi:
        if e not in met:
            for p in (63, 64):
                rows.add(members[e][p])
                met.update(int(v) for v in idx[members[e][p]])
    for e in multi[:3]:
        if cnt[e] > 128:
            rows.update((members[e][127], members[e][128]))
    assert multi and all(e in met for e in multi)
    return sorted(rows)


def test_real_streamed_skewed_m2048(real_experts):
    # the skewed prefill as benchmarked: 2048 tokens, the calibrated Zipf-shaped
    # bias (the 38 most loaded experts take half of the picks, 39 groups of more
    # than 64 rows), 96 device slots, every expert in the host arena
    bias = S.skewed_bias(S.REAL, 4, S.C4_BIAS_SCALE)
    layer = Layer(S.REAL, 1, bias=bias, router_std=0.02, max_tokens=2048, experts=real_experts, n_slots=96,
                  bind_all=False, host_arena=True)
    try:
        x = S.make_tokens(2048, S.REAL.dim, 4, index=0)
        moe.moe_reset_stats(layer.ctx)
        check_layer(layer, x, "streamed skewed m=2048", sample_rows=chunk_boundary_rows)
        st = moe.moe_get_stats(layer.ctx)
        print(f"stats {st}", flush=True)
        assert st["waves"] > 1 and st["misses"] > 0 and st["compute_ms"] > 0
    finally:
        layer.close()


def test_real_streamed_skewed_prefill(real_experts):
    # the real layer with the calibrated skewed bias, 96 device slots and every
    # expert in the host arena: several waves per call
    bias = S.skewed_bias(S.REAL, 4, S.C4_BIAS_SCALE)
    layer = Layer(S.REAL, 1, bias=bias, router_std=0.02, max_tokens=512, experts=real_experts, n_slots=96,
                  bind_all=False, host_arena=True)
    try:
        x = S.make_tokens(512, S.REAL.dim, 4, index=0)
        moe.moe_reset_stats(layer.ctx)
        check_layer(layer, x, "streamed skewed m=512", sample_rows=[0, 255, 511])
        st = moe.moe_get_stats(layer.ctx)
        print(f"stats {st}", flush=True)
        assert st["waves"] > 1 and st["misses"] > 0
    finally:
        layer.close()


def drawn_streamed(n, seed):
    from test_gpu_parity import drawn_configs
    rng = np.random.default_rng(seed)
    return [(*c, int(rng.choice([2, 3, 5, 8]))) for c in drawn_configs(n, seed)]


@pytest.mark.parametrize("dim,inter,E,k,m,shared,n_slots", drawn_streamed(8, 555))
def test_drawn_streamed(dim, inter, E, k, m, shared, n_slots):
    # drawn layer configurations with a few device slots: misses copied from the host
    # arena, waves when the picks outnumber the slots
    n_slots = min(n_slots, E)
    shape = S.LayerShape(dim, inter, E, k)
    layer = Layer(shape, 9, max_tokens=m, shared_fmt=shared, n_slots=n_slots, bind_all=False, host_arena=True)
    try:
        x = S.make_tokens(m, dim, 9, index=300 + m)
        moe.moe_reset_stats(layer.ctx)
        check_layer(layer, x, f"drawn streamed {dim}x{inter} E={E} k={k} m={m} {shared} slots={n_slots}")
        st = moe.moe_get_stats(layer.ctx)
        distinct = len(set(layer.oracle_route(x)[0].reshape(-1).tolist()))
        assert st["misses"] >= distinct - min(distinct, n_slots)
        assert st["bytes_copied"] == st["misses"] * layer.arena_src.shape[1]
        assert st["waves"] == (1 if distinct <= n_slots else -(-distinct // max(1, n_slots // 2)))
    finally:
        layer.close()
