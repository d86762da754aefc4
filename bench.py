#!/usr/bin/env python3
"""Throughput of the quantised MoE layer (C ABI, HIP kernels) on one MI355X.

Workloads (seeded synthetic inputs at the pages' DeepSeek-V4.1 layer shape:
dim 5120, inter 2304, 384 routed experts, top-6, Q2_K gate/up and Q3_K down
blocks, bf16 shared expert):
  decode  (default): m = 1 token per step; the step cycles a pool of 256 tokens
          and 4 layers' router + shared expert over one 384-expert pool, so no
          step finds its weights in the 256 MB last-level cache from the step
          before (the routed experts differ per token anyway).
  prefill: m = 512 tokens per step, uniform routing (zero bias).
A step is one moe_forward call (every kernel of the layer). Prints one JSON
line; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "MoE layer tokens/s (m=1 GEMV, m=512 MMQ) + expert-weight HBM GB/s vs peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_ffn_gemv_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(layers, tokens, experts, shape, sample):
    """The oracle, as it stands, on `sample` steps of the same workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle

    def bits(t):
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    cfg = oracle.MoeCfg(shape.dim, shape.inter, shape.n_routed, shape.topk)
    cache = {}

    def expert_bytes(e):
        if e not in cache:
            cache[e] = experts[e].cpu().numpy()
        return cache[e]

    lay = layers[0]
    shared = {"fmt": "bf16", **{k: bits(lay["shared"][k]) for k in ("w1", "w3", "w2")}}
    wr = bits(lay["wr"])
    bias = lay["bias"].cpu().numpy()
    xs = [bits(tokens[i:i + 1]) for i in range(sample)]
    # copy the picked experts out before the clock starts (they come from the GPU pool)
    for x in xs:
        idx = oracle.route(cfg, oracle.bf16_bits_to_f64(x), oracle.bf16_bits_to_f64(wr), bias)[0]
        for e in np.unique(idx):
            expert_bytes(int(e))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for x in xs:
            oracle.moe_layer(cfg, x, wr, bias, lambda e: cache[e], shared)
        dt = time.perf_counter() - t0
    return {"value": sample / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{sample} decode tokens (m=1) of layer 0: float64 numpy oracle incl. decoding the "
                      f"6 picked experts' blocks per token; {dt:.1f} s on one host core"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=("decode", "prefill"), default="decode")
    ap.add_argument("--layers", type=int, default=4, help="layers (router + shared) in rotation (decode)")
    ap.add_argument("--cpu-sample", type=int, default=2, help="oracle steps for cpu_baseline (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (no sharding, no "
              "collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_ffn_gemv_amd as moe
    import synthetic as S

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    shape = S.REAL
    decode = args.workload == "decode"
    m = 1 if decode else 512
    n_layers = args.layers if decode else 1

    t0 = time.time()
    experts = S.make_experts(shape, 1, device=dev)
    torch.cuda.synchronize()
    log(f"experts drawn in {time.time() - t0:.1f}s ({experts.numel() / 1e9:.2f} GB)")
    layers = []
    for li in range(n_layers):
        seed = 1 if li == 0 else 1000 + li
        wr, bias = S.make_router(shape, seed, 0.02, (-0.05, 0.05) if decode else None)
        sh = S.make_shared(shape, seed, "bf16")
        lay = {"wr": wr, "bias": bias, "shared": sh,
               "d_wr": wr.to(dev), "d_bias": bias.to(dev), "d_sh": {k: sh[k].to(dev) for k in ("w1", "w3", "w2")}}
        lay["w"] = moe.make_weights(lay["d_wr"], lay["d_bias"], moe.MOE_SHARED_BF16, lay["d_sh"]["w1"],
                                    lay["d_sh"]["w3"], lay["d_sh"]["w2"])
        layers.append(lay)
    pool_n = 256 if decode else 512
    tokens = S.make_tokens(pool_n, shape.dim, 1, index=0 if decode else 2)
    d_tokens = tokens.to(dev)
    cfg = moe.make_cfg(shape.dim, shape.inter, shape.n_routed, shape.topk, max_tokens=max(m, 8))
    ctx = moe.moe_create(cfg)
    moe.moe_set_slots(ctx, experts, shape.n_routed)
    for e in range(shape.n_routed):
        moe.moe_slot_bind(ctx, e, e)
    out = torch.empty((m, shape.dim), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((m, shape.topk), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, with_idx=False):
        lay = layers[i % n_layers]
        x = d_tokens[i % pool_n:i % pool_n + 1] if decode else d_tokens
        if with_idx:
            moe.moe_forward_ex(ctx, lay["w"], x, m, out, None, idx, stream)
        else:
            moe.moe_forward(ctx, lay["w"], x, m, out, stream)

    for i in range(args.warmup):
        step(i)
    rc = moe.moe_check(ctx)
    if rc != moe.MOE_OK:
        raise RuntimeError(f"warmup: {moe.strerror(rc)}")

    # distinct experts per step (prefill: algorithmic bytes depend on the routing)
    distinct = []
    if not decode:
        for i in range(min(args.steps, 4)):
            step(i, with_idx=True)
            distinct.append(len(torch.unique(idx)))
        torch.cuda.synchronize()

    # timed region: K steps bracketed by events on the launch stream
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    rc = moe.moe_check(ctx)
    if rc != moe.MOE_OK:
        raise RuntimeError(f"timed region: {moe.strerror(rc)}")

    # the same K steps again with every kernel launch bracketed by HIP events on
    # its own stream (the library records them): per-kernel durations
    moe.moe_set_profiling(ctx, True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_profiled = ev0.elapsed_time(ev1)
    ktimes = moe.moe_kernel_times(ctx)
    moe.moe_set_profiling(ctx, False)

    ms_step = ms_total / args.steps
    value = m * args.steps / (ms_total / 1e3)

    q2k_matrix = shape.inter * (shape.dim // 256) * 84
    q3k_matrix = shape.dim * (shape.inter // 256) * 110
    n_exp = shape.topk if decode else sum(distinct) / len(distinct)
    gateup_bytes = n_exp * 2 * q2k_matrix
    down_bytes = n_exp * q3k_matrix
    shared_bytes = 3 * shape.dim * shape.inter * 2

    def avg_ms(k):
        s, n = ktimes[k]
        return s / n if n else float("nan")

    ga = avg_ms("gateup")
    achieved = gateup_bytes / (ga / 1e3) / 1e9
    traffic = stored_traffic(args.workload, "gateup")
    expert_ms = sum(avg_ms(k) for k in ("gateup", "down", "shared_gateup", "shared_down"))
    expert_bytes = gateup_bytes + down_bytes + shared_bytes
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": ("decode m=1" if decode else "prefill m=512")
            + ": dim 5120, inter 2304, 384 routed experts top-6 (Q2_K gate/up, Q3_K down) x q8_1, bf16 shared",
            "m": m,
            "layers_in_rotation": n_layers,
            "token_pool": pool_n,
            "experts_per_step": n_exp,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gateup_q2k (routed gate/up GEMV + SwiGLU)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": int(gateup_bytes),
            "avg_launch_ms": round(ga, 5),
        },
        "expert_kernels": {
            "bytes_per_step": int(expert_bytes),
            "summed_ms": round(expert_ms, 5),
            "GB_per_s": round(expert_bytes / (expert_ms / 1e3) / 1e9, 1),
            "frac_of_hbm_peak": round(expert_bytes / (expert_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "layer_GB_per_s": round(expert_bytes / (ms_step / 1e3) / 1e9, 1),
        "ms_per_step_with_kernel_events": round(ms_profiled / args.steps, 5),
        "kernel_timing": "per-kernel HIP events (recorded by the library on each launch's stream) over a "
                         "replay of the same steps right after the timed region",
        "kernel_avg_ms": {k: round(avg_ms(k), 5) for k in ktimes if ktimes[k][1]},
    }
    if args.cpu_sample > 0 and decode:
        log("cpu baseline: running the oracle")
        result["cpu_baseline"] = cpu_baseline(layers, tokens, experts, shape, args.cpu_sample)
    else:
        result["cpu_baseline"] = None
    moe.moe_destroy(ctx)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
