"""A MoE layer built from the seeded synthetic inputs, resident on a GPU and
driven through the C ABI; plus the oracle's view of the same bytes.

Used by the GPU tests and by the CPU-baseline leg of bench.py's reference
checks. The oracle always reads the exact bytes the device holds (blocks drawn
on the GPU are copied back).
"""
import time

import numpy as np
import torch

import mixture_experts_ffn_gemv_amd as moe
import synthetic as S


def bits(t):
    """bf16 tensor (any device) -> uint16 numpy bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


class Layer:
    def __init__(self, shape, seed, *, shared_fmt="bf16", bias=(-0.1, 0.1), router_std=0.05, max_tokens=8,
                 expert_device="cpu", gate_temp=1.0, norm=True, route_scale=1.5, limit=10.0, bind_all=True,
                 n_slots=None, experts=None, host_arena=False, dispatch=None, expert_fmt="kquant",
                 verbose=False):
        self.shape = shape
        self.dev = torch.device("cuda")
        t0 = time.time()
        self.wr, self.bias = S.make_router(shape, seed, router_std, bias)
        self.expert_fmt = expert_fmt
        self.arena_src = (experts if experts is not None
                          else S.make_experts(shape, seed, device=expert_device, fmt=expert_fmt))
        self.shared = None if shared_fmt == "none" else S.make_shared(shape, seed, shared_fmt)
        self.cfg = moe.make_cfg(shape.dim, shape.inter, shape.n_routed, shape.topk, gate_temp=gate_temp,
                                norm_topk_prob=norm, route_scale=route_scale, swiglu_limit=limit,
                                max_tokens=max_tokens,
                                expert_fmt=moe.MOE_EXPERT_MXFP4 if expert_fmt == "fp4" else moe.MOE_EXPERT_KQUANT)
        self.ocfg_kw = dict(gate_temp=gate_temp, norm_topk_prob=norm, route_scale=route_scale,
                            swiglu_limit=limit, expert_fmt=expert_fmt)
        self.ctx = moe.moe_create(self.cfg)
        if dispatch is not None:
            moe.moe_set_dispatch(self.ctx, dispatch)
        self.n_slots = n_slots or shape.n_routed
        # the library reads slots in its panel layout; the oracle reads arena_src (plain GGUF rows)
        packed = moe.pack_experts(self.cfg, self.arena_src.to(self.dev))
        if self.n_slots == shape.n_routed:
            self.arena = packed
        else:
            self.arena = torch.zeros((self.n_slots, self.arena_src.shape[1]), dtype=torch.uint8, device=self.dev)
        moe.moe_set_slots(self.ctx, self.arena, self.n_slots)
        if bind_all and self.n_slots == shape.n_routed:
            for e in range(shape.n_routed):
                moe.moe_slot_bind(self.ctx, e, e)
        self.host = None
        if host_arena:
            # every expert in page-locked host memory (a new pinned tensor, not a registered one)
            self.host = torch.empty(self.arena_src.shape, dtype=torch.uint8, pin_memory=True)
            self.host.copy_(packed)
            moe.moe_set_host_arena(self.ctx, self.host, self.arena_src.shape[1])
        self.d_wr = self.wr.to(self.dev)
        self.d_bias = self.bias.to(self.dev)
        self.d_shared = None
        fmt = moe.MOE_SHARED_NONE
        if self.shared is not None:
            if shared_fmt == "bf16":
                self.d_shared = {k: self.shared[k].to(self.dev) for k in ("w1", "w3", "w2")}
                fmt = moe.MOE_SHARED_BF16
            else:
                slot = torch.empty(self.shared["slot"].shape, dtype=torch.uint8, device=self.dev)
                # a K-quant slice, packed with the K-quant layout whatever the routed format
                kcfg = moe.make_cfg(shape.dim, shape.inter, shape.n_routed, shape.topk, max_tokens=max_tokens)
                moe.moe_pack_expert(kcfg, self.shared["slot"].to(self.dev), slot)
                _, o1, o3, o2 = S.expert_layout(shape)
                self.d_shared = {"slot": slot, "w1": slot[o1:o3], "w3": slot[o3:o2], "w2": slot[o2:]}
                fmt = moe.MOE_SHARED_KQUANT
        sw = self.d_shared or {}
        self.w = moe.make_weights(self.d_wr, self.d_bias, fmt, sw.get("w1"), sw.get("w3"), sw.get("w2"))
        if verbose:
            print(f"layer ready in {time.time() - t0:.1f}s", flush=True)

    def close(self):
        if self.ctx is not None:
            moe.moe_destroy(self.ctx)
            self.ctx = None
        self.arena = None   # the packed copy (the caller may hold the plain one)

    def forward(self, x, m=None, stream=None):
        m = x.shape[0] if m is None else m
        k = self.shape.topk
        out = torch.empty((m, self.shape.dim), dtype=torch.bfloat16, device=self.dev)
        gw = torch.empty((m, k), dtype=torch.float32, device=self.dev)
        idx = torch.empty((m, k), dtype=torch.int32, device=self.dev)
        moe.moe_forward_ex(self.ctx, self.w, x, m, out, gw, idx, stream)
        return out, gw, idx

    def check(self):
        return moe.moe_check(self.ctx)

    # ------------------------------------------------------------------ oracle side
    def oracle_cfg(self):
        import oracle
        return oracle.MoeCfg(self.shape.dim, self.shape.inter, self.shape.n_routed, self.shape.topk, **self.ocfg_kw)

    def oracle_shared(self):
        if self.shared is None:
            return None
        if self.shared["fmt"] == "bf16":
            return {"fmt": "bf16", **{k: bits(self.shared[k]) for k in ("w1", "w3", "w2")}}
        return {"fmt": "kquant", "slot": self.shared["slot"].numpy()}

    def expert_bytes(self, e):
        return self.arena_src[e].cpu().numpy()

    def oracle(self, x_rows):
        import oracle
        return oracle.moe_layer(self.oracle_cfg(), bits(x_rows), bits(self.wr), self.bias.numpy(),
                                self.expert_bytes, self.oracle_shared())

    def oracle_parallel(self, x_rows):
        """As oracle(), with the rows dealt out to worker processes (real-shape
        layers, many sampled rows)."""
        import oracle
        from oracle_pool import oracle_rows
        picks = self.oracle_route(x_rows)[0]
        cfg = self.oracle_cfg()
        cfg_args = (cfg.dim, cfg.inter, cfg.n_routed, cfg.topk)
        return oracle_rows(cfg_args, self.ocfg_kw, bits(x_rows), bits(self.wr), self.bias.numpy(),
                           self.expert_bytes, self.oracle_shared(), picks)

    def oracle_route(self, x_rows):
        import oracle
        x = oracle.bf16_bits_to_f64(bits(x_rows))
        wr = oracle.bf16_bits_to_f64(bits(self.wr))
        return oracle.route(self.oracle_cfg(), x, wr, self.bias.numpy())


def compare_routing(idx_gpu, gw_gpu, idx_ref, g_ref, keys_ref, gap=1e-5):
    """Indices bit-exact except where the pages' near-tie exemption applies:
    a set difference only when key_(k) - key_(k+1) < gap, an order swap only
    between keys closer than gap (gaps measured on the oracle's float64 keys).
    Returns the number of exempted tokens; raises AssertionError otherwise."""
    idx_gpu = np.asarray(idx_gpu)
    exempt = 0
    k = idx_ref.shape[1]
    for t in range(idx_ref.shape[0]):
        a, b = list(idx_gpu[t]), list(idx_ref[t])
        if a == b:
            assert np.allclose(gw_gpu[t], g_ref[t], rtol=1e-5, atol=1e-7), (t, gw_gpu[t], g_ref[t])
            continue
        keys = keys_ref[t]
        srt = np.sort(keys)[::-1]
        if set(a) != set(b):
            assert k < len(keys) and srt[k - 1] - srt[k] < gap, (t, a, b, srt[k - 1] - srt[k])
        else:
            for i in range(k):
                if a[i] != b[i]:
                    assert abs(keys[a[i]] - keys[b[i]]) < gap, (t, a, b)
        exempt += 1
    return exempt
