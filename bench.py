#!/usr/bin/env python3
"""Throughput of the quantised MoE layer (C ABI, HIP kernels) on one MI355X.

Workloads (seeded synthetic inputs at the pages' DeepSeek-V4.1 layer shape:
dim 5120, inter 2304, 384 routed experts, top-6, Q2_K gate/up and Q3_K down
blocks; router weights ~N(0, 0.02); expert weights ~N(0, 0.02) before
quantisation; tokens ~N(0, 1) in bf16):
  decode       m = 1 per step, bf16 shared expert, bias ~U(-0.05, 0.05). The
               step cycles a pool of 256 tokens and 4 layers' router + shared
               expert over one 384-expert pool, so no step finds its weights in
               the 256 MB last-level cache from the step before (the routed
               experts differ per token anyway). The headline line.
  small        m = 8 independent tokens per step, K-quant shared expert.
  prefill      m = 512 tokens per step, uniform routing (zero bias).
  prefill_hot  m = 512 with bias +100 on six fixed experts: every token picks
               them, six groups of 512 rows, the shape where int8 MFMA binds.
  skewed       m = 2048 with a Zipf(1.1)-shaped bias (calibrated so the 38
               most loaded experts take half of the assignments), only 96
               device slots, every expert in a page-locked host arena: each
               call streams its missing experts in over the host link (least
               recently used slots reused, waves when the picks outnumber the
               slots). The LRU is warmed with 3 untimed calls.
A step is one moe_forward call (every kernel of the layer). Prints one JSON
line for the chosen workload; with the decode headline the others are
summarised under "workloads" (unless --no-extra). Progress goes to stderr.
At m <= 8 the line also gives the median, p10 and p90 of single calls, each
between its own event pair: cold (the rotation above) and warm (one token
through one layer again and again, so the last-level cache serves what it
holds of that layer).

--traffic-from FETCH.csv WRITE.csv turns two rocprofv3 --pmc counter files
(FETCH_SIZE, then WRITE_SIZE, of a run with --copy-calibration) into HBM bytes
per launch of the workload's dominant kernel and stores them in
profiles/traffic.json; no GPU is used for that.
"""
import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
I8_PEAK_OPS = 5.0e15            # MI355X dense int8 MFMA
METRIC = "MoE layer tokens/s (m=1 GEMV, m=512 MMQ) + expert-weight HBM GB/s vs peak"
COPY_BYTES = 1 << 30            # the calibration copy reads and writes 1 GiB
HOT_EXPERTS = (5, 77, 140, 203, 266, 329)

WORKLOADS = {
    "decode": dict(m=1, layers=4, bias=(-0.05, 0.05), shared="bf16", pool=256,
                   desc="decode m=1 (GEMV path), bf16 shared expert"),
    "small": dict(m=8, layers=4, bias=(-0.05, 0.05), shared="kquant", pool=256,
                  desc="small batch m=8 (GEMV path), K-quant shared expert"),
    "decode_fp4": dict(m=1, layers=4, bias=(-0.05, 0.05), shared="bf16", pool=256, experts="fp4",
                       desc="decode m=1, MXFP4 routed experts (e2m1 codes, E8M0 scale per 32 weights) on bf16 "
                            "activations, bf16 shared expert"),
    "prefill": dict(m=512, layers=1, bias=None, shared="bf16", pool=512,
                    desc="prefill m=512 (MMQ path), uniform routing, bf16 shared expert"),
    "prefill_mixed": dict(m=512, layers=1, bias=None, shared="bf16", pool=512, dispatch="mixed",
                          desc="prefill m=512 with groups of <= 8 rows on the GEMV kernels and larger ones on "
                               "MMQ, uniform routing, bf16 shared expert"),
    "prefill_fp4": dict(m=512, layers=1, bias=None, shared="bf16", pool=512, experts="fp4",
                        desc="prefill m=512, MXFP4 routed experts on bf16 activations, uniform routing, bf16 "
                             "shared expert"),
    "prefill_hot": dict(m=512, layers=1, bias="hot", shared="bf16", pool=512,
                        desc="prefill m=512 (MMQ path), 6 hot experts take every token, bf16 shared expert"),
    "skewed": dict(m=2048, layers=1, bias="skewed", shared="bf16", pool=2048, slots=96,
                   desc="skewed prefill m=2048 (MMQ path), 96 device slots, misses streamed from a pinned host "
                        "arena, bf16 shared expert"),
}
# the kernel each workload's roofline object describes, and its name in rocprofv3
DOMINANT = {
    "decode": ("gateup", r"^(void )?moe::gateup_q8_kernel\b"),
    "small": ("gateup", r"^(void )?moe::gateup_q8_kernel\b"),
    "decode_fp4": ("gateup", r"^void moe::fp4_gemv_kernel<2, 1, 5>"),
    "prefill_fp4": ("gateup", r"^void moe::fp4_mmq_kernel<1, false>"),  # the <= 16-row class
    "prefill": ("gateup", r"^void moe::mmq_gateup_q2k_kernel<1>"),      # the <= 16-row class
    "prefill_mixed": ("gateup", r"^void moe::gateup_q2k_kernel<8>"),    # the groups of <= 8 rows
    "prefill_hot": ("gateup", r"^void moe::mmq_gateup_q2k_kernel<4>"),  # the 64-row class
    "skewed": ("gateup", r"^void moe::mmq_gateup_q2k_kernel<4>"),
}
COPY_KERNEL = r"neg_kernel"


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


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def stored_traffic(workload):
    """HBM bytes per launch of the dominant kernel from rocprofv3 counters, if
    they were taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        ent = json.load(f).get(workload)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def traffic_from(fetch_csv, write_csv, workload):
    """Scale the per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the dominant
    kernel by what the same counters read for the 1 GiB calibration copy."""
    kname = re.compile(DOMINANT[workload][1])
    copy = re.compile(COPY_KERNEL)

    def per_dispatch(path, counter):
        ker, cal = {}, {}
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        # the calibration copy: the largest grid among the copy kernel's dispatches
        copy_grid = max(int(r["Grid_Size"]) for r in rows if copy.search(r["Kernel_Name"]))
        for row in rows:
            v = float(row["Counter_Value"])
            key = row["Dispatch_Id"]
            if kname.search(row["Kernel_Name"]):
                ker[key] = ker.get(key, 0.0) + v
            elif copy.search(row["Kernel_Name"]) and int(row["Grid_Size"]) == copy_grid:
                cal[key] = cal.get(key, 0.0) + v
        if not ker or not cal:
            raise SystemExit(f"{path}: no {counter} rows for the kernel ({len(ker)}) or the copy ({len(cal)})")
        return sum(ker.values()) / len(ker), sum(cal.values()) / len(cal), len(ker)

    f_k, f_c, n_f = per_dispatch(fetch_csv, "FETCH_SIZE")
    w_k, w_c, n_w = per_dispatch(write_csv, "WRITE_SIZE")
    copy_kib = COPY_BYTES / 1024.0
    f_scale, w_scale = copy_kib / f_c, copy_kib / w_c
    fetch_b = f_k * 1024.0 * f_scale
    write_b = w_k * 1024.0 * w_scale
    rec = {}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f)
    rec[workload] = {
        "kernel": DOMINANT[workload][1],
        "fetch_kib_per_dispatch": round(f_k, 1), "write_kib_per_dispatch": round(w_k, 1),
        "dispatches": [n_f, n_w],
        "copy_fetch_kib": round(f_c, 1), "copy_write_kib": round(w_c, 1),
        "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
        "bytes_per_launch": int(fetch_b + write_b),
        "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
        "source_hash": kernel_source_hash(),
    }
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(rec[workload]))


CPU_WORKERS_MAX = 16   # the host share of one GPU


def _oracle_token(args):
    """One decode token through the oracle's whole layer (a worker process)."""
    from threadpoolctl import threadpool_limits

    import oracle
    cfg_args, x, wr, bias, experts, shared = args
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.moe_layer(oracle.MoeCfg(*cfg_args), x, wr, bias, lambda e: experts[e], shared)
        return time.perf_counter() - t0


def _oracle_group(args):
    """One expert's group of a prefill batch: decode its blocks, run its rows (a worker process)."""
    from threadpoolctl import threadpool_limits

    import oracle
    cfg_args, raw, x_rows = args
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        cfg = oracle.MoeCfg(*cfg_args)
        w1, w3, w2 = oracle.slot_matrices(cfg, raw)
        oracle.expert_ffn_kquant(x_rows, w1, w3, w2, cfg.swiglu_limit)
        return time.perf_counter() - t0


def _warm(_):
    """Start a worker: import what the tasks need (not timed)."""
    from threadpoolctl import threadpool_limits  # noqa: F401

    import oracle  # noqa: F401
    time.sleep(0.5)
    return os.getpid()


def _pool(workers):
    import concurrent.futures
    import multiprocessing
    return concurrent.futures.ProcessPoolExecutor(max_workers=workers, mp_context=multiprocessing.get_context("spawn"))


def cpu_baseline(lay, tokens, experts, shape, decode_tokens=None, prefill_groups=32):
    """The oracle, as it stands, on the host's cores (worker processes, one BLAS
    thread each), on bounded samples of the decode and prefill workloads."""
    import platform

    import numpy as np
    import torch

    import oracle
    import synthetic as S

    def bits(t):
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    workers = max(1, min(CPU_WORKERS_MAX, os.cpu_count() or 1))
    n_dec = decode_tokens or workers
    cfg = oracle.MoeCfg(shape.dim, shape.inter, shape.n_routed, shape.topk)
    cfg_args = (shape.dim, shape.inter, shape.n_routed, shape.topk)
    cpu_model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name"))
    except (OSError, StopIteration):
        pass

    # decode: n_dec tokens of the same pool, one whole-layer oracle call each
    shared = {"fmt": "bf16", **{k: bits(lay["shared"][k]) for k in ("w1", "w3", "w2")}}
    wr, bias = bits(lay["wr"]), lay["bias"].cpu().numpy()
    wr64 = oracle.bf16_bits_to_f64(wr)
    tasks = []
    for i in range(n_dec):
        x = bits(tokens[i:i + 1])
        picks = oracle.route(cfg, oracle.bf16_bits_to_f64(x), wr64, bias)[0]
        tasks.append((cfg_args, x, wr, bias, {int(e): experts[int(e)].cpu().numpy() for e in np.unique(picks)},
                      shared))
    pool = _pool(workers)
    list(pool.map(_warm, range(workers)))   # start the workers (imports) before the clock
    t0 = time.perf_counter()
    list(pool.map(_oracle_token, tasks))
    dt_dec = time.perf_counter() - t0
    del tasks

    # prefill m = 512 (uniform routing): the routing and the bf16 shared expert for all
    # 512 tokens in this process (BLAS on every core), and a sample of the expert
    # groups (every 12th expert id) in the workers; the whole is the sample scaled by
    # the groups left out
    wr_p, bias_p = S.make_router(shape, 1, 0.02, None)
    sh_p = S.make_shared(shape, 1, "bf16")
    xp = bits(S.make_tokens(512, shape.dim, 1, index=2))
    x64 = oracle.bf16_bits_to_f64(xp)
    t0 = time.perf_counter()
    idx = oracle.route(cfg, x64, oracle.bf16_bits_to_f64(bits(wr_p)), bias_p.numpy())[0]
    oracle.shared_ffn_bf16(x64, *(oracle.bf16_bits_to_f64(bits(sh_p[k])) for k in ("w1", "w3", "w2")),
                           cfg.swiglu_limit)
    dt_main = time.perf_counter() - t0
    groups = [e for e in range(0, shape.n_routed, max(1, shape.n_routed // prefill_groups)) if (idx == e).any()]
    all_groups = len(np.unique(idx))
    x32 = x64.astype(np.float32)
    gtasks = [(cfg_args, experts[e].cpu().numpy(), x32[np.nonzero((idx == e).any(axis=1))[0]]) for e in groups]
    t0 = time.perf_counter()
    list(pool.map(_oracle_group, gtasks))
    dt_groups = time.perf_counter() - t0
    pool.shutdown()
    est_prefill = dt_main + dt_groups * all_groups / len(groups)
    return {
        "value": round(n_dec / dt_dec, 4), "unit": "tokens/s", "cores": workers, "kind": "oracle",
        "sample": f"{n_dec} decode tokens (m=1) of the headline layer, each one call of the float64 numpy "
                  f"oracle's whole layer (decoding its 6 picked experts' blocks) in {workers} worker processes "
                  f"(one BLAS thread each): {dt_dec:.1f} s wall; host: {os.cpu_count()} logical CPUs, {cpu_model}",
        "prefill_m512": {
            "value": round(512 / est_prefill, 3), "unit": "tokens/s",
            "sample": f"prefill m=512 (uniform routing): routing and bf16 shared expert for all 512 tokens in one "
                      f"process with BLAS on every core ({dt_main:.1f} s), plus {len(groups)} of the "
                      f"{all_groups} expert groups (every 12th expert id, all its rows) decoded and run in "
                      f"{workers} workers ({dt_groups:.1f} s); the groups' time scaled by {all_groups}/"
                      f"{len(groups)}: {est_prefill:.1f} s per 512-token step",
        },
    }


class Bench:
    def __init__(self, shape):
        import torch

        import mixture_experts_ffn_gemv_amd as moe
        import synthetic as S
        self.torch, self.moe, self.S = torch, moe, S
        self.shape = shape
        self.dev = torch.device("cuda:0")
        t0 = time.time()
        self.experts = S.make_experts(shape, 1, device=self.dev)   # plain GGUF row order (the oracle's view)
        self.cfg0 = moe.make_cfg(shape.dim, shape.inter, shape.n_routed, shape.topk)
        self.packed = moe.pack_experts(self.cfg0, self.experts)      # the library's slot layout
        torch.cuda.synchronize()
        log(f"experts drawn in {time.time() - t0:.1f}s ({self.experts.numel() / 1e9:.2f} GB)")
        self.slot_bytes = self.experts.shape[1]
        self._fp4 = None

    def fp4_arena(self):
        """The 384 experts in MXFP4 (7.2 GB) in the library's tiled slot layout, drawn
        from the same seeds on first use."""
        if self._fp4 is None:
            t0 = time.time()
            plain = self.S.make_experts(self.shape, 1, device=self.dev, fmt="fp4")
            shape, moe = self.shape, self.moe
            cfg = moe.make_cfg(shape.dim, shape.inter, shape.n_routed, shape.topk, expert_fmt=moe.MOE_EXPERT_MXFP4)
            self._fp4 = moe.pack_experts(cfg, plain)
            self.torch.cuda.synchronize()
            del plain
            log(f"MXFP4 experts drawn in {time.time() - t0:.1f}s ({self._fp4.numel() / 1e9:.2f} GB)")
        return self._fp4

    def layers(self, wl):
        torch, moe, S, shape = self.torch, self.moe, self.S, self.shape
        spec = WORKLOADS[wl]
        out = []
        for li in range(spec["layers"]):
            seed = 1 if li == 0 else 1000 + li
            if spec["bias"] == "hot":
                b = torch.zeros(shape.n_routed, dtype=torch.float32)
                b[list(HOT_EXPERTS)] = 100.0
                wr, bias = S.make_router(shape, seed, 0.02, b)
            elif spec["bias"] == "skewed":
                wr, bias = S.make_router(shape, seed, 0.02, S.skewed_bias(shape, 4, S.C4_BIAS_SCALE))
            else:
                wr, bias = S.make_router(shape, seed, 0.02, spec["bias"])
            sh = S.make_shared(shape, seed, spec["shared"])
            lay = {"wr": wr, "bias": bias, "shared": sh, "d_wr": wr.to(self.dev), "d_bias": bias.to(self.dev)}
            if spec["shared"] == "bf16":
                lay["d_sh"] = {k: sh[k].to(self.dev) for k in ("w1", "w3", "w2")}
                lay["w"] = moe.make_weights(lay["d_wr"], lay["d_bias"], moe.MOE_SHARED_BF16, lay["d_sh"]["w1"],
                                            lay["d_sh"]["w3"], lay["d_sh"]["w2"])
            else:
                slot = torch.empty_like(sh["slot"], device=self.dev)
                moe.moe_pack_expert(self.cfg0, sh["slot"].to(self.dev), slot)
                _, o1, o3, o2 = S.expert_layout(shape)
                lay["d_sh"] = {"slot": slot}
                lay["w"] = moe.make_weights(lay["d_wr"], lay["d_bias"], moe.MOE_SHARED_KQUANT, slot[o1:],
                                            slot[o3:], slot[o2:])
            out.append(lay)
        return out

    def run(self, wl, steps, warmup, copy_calibration=False):
        torch, moe, S, shape = self.torch, self.moe, self.S, self.shape
        spec = WORKLOADS[wl]
        m, pool_n = spec["m"], spec["pool"]
        layers = self.layers(wl)
        n_layers = len(layers)
        if wl == "skewed":
            tokens = S.make_tokens(pool_n, shape.dim, 4, index=0)
        else:
            tokens = S.make_tokens(pool_n, shape.dim, 1, index={"decode": 0, "small": 3}.get(wl, 2))
        d_tokens = tokens.to(self.dev)
        fp4 = spec.get("experts") == "fp4"
        cfg = moe.make_cfg(shape.dim, shape.inter, shape.n_routed, shape.topk, max_tokens=max(m, 8),
                           expert_fmt=moe.MOE_EXPERT_MXFP4 if fp4 else moe.MOE_EXPERT_KQUANT)
        ctx = moe.moe_create(cfg)
        if spec.get("dispatch") == "mixed":
            moe.moe_set_dispatch(ctx, moe.MOE_DISPATCH_MIXED)
        streamed = "slots" in spec
        if streamed:
            # a small device arena; every expert in page-locked host memory
            slot_arena = torch.empty((spec["slots"], self.slot_bytes), dtype=torch.uint8, device=self.dev)
            host = self.pinned_experts()
            moe.moe_set_slots(ctx, slot_arena, spec["slots"])
            moe.moe_set_host_arena(ctx, host, self.slot_bytes)
        else:
            moe.moe_set_slots(ctx, self.fp4_arena() if fp4 else self.packed, shape.n_routed)
            for e in range(shape.n_routed):
                moe.moe_slot_bind(ctx, e, e)
        out = torch.empty((m, shape.dim), dtype=torch.bfloat16, device=self.dev)
        idx = torch.empty((m, shape.topk), dtype=torch.int32, device=self.dev)
        stream = torch.cuda.current_stream()
        if copy_calibration:
            # a plain elementwise copy (negation) of known size, for scaling the
            # HBM byte counters of rocprofv3 --pmc runs
            src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=self.dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                torch.neg(src, out=dst)
            torch.cuda.synchronize()
            del src, dst

        def xs(i):
            if m == pool_n:
                return d_tokens
            j = (i * m) % pool_n
            return d_tokens[j:j + m]

        def step(i, with_idx=False):
            lay = layers[i % n_layers]
            if with_idx:
                moe.moe_forward_ex(ctx, lay["w"], xs(i), m, out, None, idx, stream)
            else:
                moe.moe_forward(ctx, lay["w"], xs(i), m, out, stream)

        for i in range(warmup):
            step(i)
        rc = moe.moe_check(ctx)
        if rc != moe.MOE_OK:
            raise RuntimeError(f"{wl} warmup: {moe.strerror(rc)}")
        moe.moe_reset_stats(ctx)

        # timed region: K steps bracketed by events on the launch stream
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(steps):
            step(warmup + i)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_total = ev0.elapsed_time(ev1)
        rc = moe.moe_check(ctx)
        if rc != moe.MOE_OK:
            raise RuntimeError(f"{wl} timed region: {moe.strerror(rc)}")
        stats = moe.moe_get_stats(ctx)

        # decode: the same steps replayed from one HIP graph holding a forward of every
        # layer in the rotation (each layer reads its own fixed input buffer); before
        # each replay one copy fills the buffers with the next tokens of the pool
        graph_ms = None
        if m <= 8 and not streamed:
            x_static = torch.empty((n_layers, m, shape.dim), dtype=torch.bfloat16, device=self.dev)
            out_static = torch.empty((n_layers, m, shape.dim), dtype=torch.bfloat16, device=self.dev)
            rounds = (steps + n_layers - 1) // n_layers
            w_rounds = max(1, (warmup + n_layers - 1) // n_layers)
            inputs = [torch.stack([xs(r * n_layers + li) for li in range(n_layers)])
                      for r in range(w_rounds + rounds)]
            x_static.copy_(inputs[0])
            for li, lay in enumerate(layers):
                moe.moe_forward(ctx, lay["w"], x_static[li], m, out_static[li])
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for li, lay in enumerate(layers):
                    moe.moe_forward(ctx, lay["w"], x_static[li], m, out_static[li])
            for r in range(w_rounds):
                x_static.copy_(inputs[r])
                g.replay()
            torch.cuda.synchronize()
            gs = torch.cuda.current_stream()
            ev0.record(gs)
            for r in range(rounds):
                x_static.copy_(inputs[w_rounds + r])
                g.replay()
            ev1.record(gs)
            torch.cuda.synchronize()
            graph_ms = ev0.elapsed_time(ev1) / (rounds * n_layers)
            rc = moe.moe_check(ctx)
            if rc != moe.MOE_OK:
                raise RuntimeError(f"{wl} graph replay: {moe.strerror(rc)}")
            del g

        # the same K steps again with every kernel launch bracketed by HIP events on
        # its own stream (the library records them): per-kernel durations
        moe.moe_set_profiling(ctx, True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(steps):
            step(warmup + i)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_profiled = ev0.elapsed_time(ev1)
        ktimes = moe.moe_kernel_times(ctx)
        moe.moe_set_profiling(ctx, False)

        # one event pair per call: the spread of single calls with the rotation above
        # (cold: each call's experts, router and shared expert mostly come from HBM), and
        # of the same token through the same layer again and again (warm: what the 256 MB
        # last-level cache holds of that layer serves the repeats)
        per_call = None
        if m <= 8 and not streamed:
            def call_times(fn, n):
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(n)]
                torch.cuda.synchronize()
                for i, (a, b) in enumerate(evs):
                    a.record(stream)
                    fn(i)
                    b.record(stream)
                torch.cuda.synchronize()
                t = sorted(a.elapsed_time(b) for a, b in evs)
                pick = lambda q: round(t[min(n - 1, int(q * (n - 1) + 0.5))], 5)
                return {"median_ms": pick(0.5), "p10_ms": pick(0.1), "p90_ms": pick(0.9), "calls": n}
            n_calls = max(10, min(steps, 200))
            cold = call_times(lambda i: step(warmup + i), n_calls)
            x0 = xs(0)
            warm = call_times(lambda i: moe.moe_forward(ctx, layers[0]["w"], x0, m, out, stream), n_calls)
            if moe.moe_check(ctx) != moe.MOE_OK:
                raise RuntimeError(f"{wl} per-call timing: {moe.strerror(moe.moe_check(ctx))}")
            per_call = {"cold": cold, "warm": warm,
                        "note": "one event pair per call; cold: the rotation of the timed region (tokens from "
                                "the pool, layers in turn); warm: one token through one layer repeatedly"}

        # where a bf16 shared expert's rows run in a call of m tokens (the library's plan)
        plan = moe.moe_plan_call(ctx, m, moe.MOE_SHARED_BF16 if spec["shared"] == "bf16" else moe.MOE_SHARED_KQUANT)
        # distinct experts per step (the algorithmic bytes follow the routing), untimed
        distinct = []
        for i in range(min(steps, 64)):
            step(warmup + i, with_idx=True)
            distinct.append(len(torch.unique(idx)))
        torch.cuda.synchronize()
        moe.moe_destroy(ctx)

        def avg_ms(k):   # per step: a class may launch several kernels per call
            s, n = ktimes[k]
            return s / steps if n else 0.0

        ms_step = ms_total / steps
        expert_b = moe.moe_expert_layout(cfg)[0]
        n_exp = sum(distinct) / len(distinct)
        q2k_matrix = (S.mxfp4_bytes(shape.inter, shape.dim) if fp4 else shape.inter * (shape.dim // 256) * 84)
        shared_b = 3 * shape.dim * shape.inter * 2 if spec["shared"] == "bf16" else expert_b
        routed_b = n_exp * expert_b
        expert_bytes = routed_b + shared_b
        router_b = shape.n_routed * shape.dim * 2
        # the bf16 shared expert's down rows that ride in the routed gate/up launch
        # (moe_plan_call: at m <= 8 with K-quant experts, part of them)
        sh_in_gateup = plan["shared_rows_gateup"] * shape.inter * 2 if spec["shared"] == "bf16" else 0
        # Every figure below sets bytes against the time of the kernels that read them.
        # The routed gate/up and down kernels read the picked experts (and a K-quant
        # shared expert's rows, which ride in them); a bf16 shared expert rides in the
        # routing launches at m <= 8 and has kernels of its own above 8 tokens, so the
        # whole-layer figure takes every weight byte over every kernel of the step.
        routed_k_bytes = routed_b + (shared_b if spec["shared"] == "kquant" else 0) + sh_in_gateup
        routed_k_ms = avg_ms("gateup") + avg_ms("down")
        all_k_ms = sum(avg_ms(k) for k in ktimes if ktimes[k][1])
        gateup_bytes = (n_exp * 2 * q2k_matrix + (2 * q2k_matrix if spec["shared"] == "kquant" else 0)
                        + sh_in_gateup)
        ga = avg_ms("gateup")
        res = {
            "workload": wl,
            "config": spec["desc"],
            "m": m,
            "steps": steps,
            "warmup": warmup,
            "ms_per_step": round(ms_step, 5),
            "tokens_per_s": round(m * steps / (ms_total / 1e3), 2),
            "layers_in_rotation": n_layers,
            "token_pool": pool_n,
            "experts_per_step": n_exp,
            "expert_weight_bytes_per_step": int(expert_bytes),
            "routed_kernels": {
                "kernels": "gateup + down (and the shared rows riding in them)",
                "bytes_per_step": int(routed_k_bytes),
                "summed_ms": round(routed_k_ms, 5),
                "GB_per_s": round(routed_k_bytes / (routed_k_ms / 1e3) / 1e9, 1),
                "frac_of_hbm_peak": round(routed_k_bytes / (routed_k_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            },
            "all_kernels": {
                "kernels": "every kernel of the step",
                "weight_bytes_per_step": int(expert_bytes + router_b),
                "summed_ms": round(all_k_ms, 5),
                "GB_per_s": round((expert_bytes + router_b) / (all_k_ms / 1e3) / 1e9, 1),
                "frac_of_hbm_peak": round((expert_bytes + router_b) / (all_k_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            },
            "layer_expert_GB_per_s": round(expert_bytes / (ms_step / 1e3) / 1e9, 1),
            "layer_all_GB_per_s": round((expert_bytes + router_b) / (ms_step / 1e3) / 1e9, 1),
            "layer_frac_of_hbm_peak": round(expert_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "ms_per_step_with_kernel_events": round(ms_profiled / steps, 5),
            "kernel_avg_ms": {k: round(avg_ms(k), 5) for k in ktimes if ktimes[k][1]},
            "gateup_bytes_per_launch": int(gateup_bytes),
            "shared_rows_in_gateup": int(plan["shared_rows_gateup"]) if spec["shared"] == "bf16" else 0,
            "gateup_avg_launch_ms": round(ga, 5),
            "gateup_GB_per_s": round(gateup_bytes / (ga / 1e3) / 1e9, 1),
            # the routed experts' W1 / W3 blocks alone over the same launch time (the
            # shared rows riding in the launch not counted)
            "gateup_routed_only_GB_per_s": round(n_exp * 2 * q2k_matrix / (ga / 1e3) / 1e9, 1),
            "plan": plan,
            "near_ties": {"tokens": int(stats["near_ties"]), "of_tokens": m * steps,
                          "rule": "k-th largest key minus the largest key left out < 1e-5 (device f32 keys)"},
        }
        if per_call is not None:
            res["per_call"] = per_call
        if graph_ms is not None:
            res["graph_replay"] = {
                "ms_per_step": round(graph_ms, 5),
                "tokens_per_s": round(m / (graph_ms / 1e3), 2),
                "layer_expert_GB_per_s": round(expert_bytes / (graph_ms / 1e3) / 1e9, 1),
                "note": "one HIP graph holding a forward of each layer in the rotation; one copy per replay "
                        "fills the layers' input buffers with the next tokens (copy included in the time)",
            }
        if m > 8:
            # useful int8 products of the routed experts: 2 ops per multiply-add,
            # gate + up (2 I D) and down (D I) per pick
            ops = 2.0 * m * shape.topk * 3 * shape.dim * shape.inter
            mmq_ms = avg_ms("gateup") + avg_ms("down")
            res["routed_int8_ops_per_step"] = ops
            res["mmq_ms"] = round(mmq_ms, 5)
            res["mmq_i8_TOPS"] = round(ops / (mmq_ms / 1e3) / 1e12, 1)
            res["mmq_i8_mfma_util"] = round(ops / (mmq_ms / 1e3) / I8_PEAK_OPS, 4)
            res["mmq_routed_GB_per_s"] = round(routed_b / (mmq_ms / 1e3) / 1e9, 1)
            res["mmq_frac_of_hbm_peak"] = round(routed_b / (mmq_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
        if streamed:
            calls = max(1, stats["calls"])
            link = stats["bytes_copied"] / (ms_total / 1e3) / 1e9
            res["streaming"] = {
                "device_slots": spec["slots"],
                "hits_per_call": stats["hits"] / calls,
                "misses_per_call": stats["misses"] / calls,
                "waves_per_call": stats["waves"] / calls,
                "bytes_copied_per_call": stats["bytes_copied"] / calls,
                "route_readback_ms_per_call": round(stats["route_ms"] / calls, 4),
                "copy_ms_per_call": round(stats["fetch_ms"] / calls, 4),
                "link_GB_per_s": round(link, 2),
                "pinned_copy_peak_GB_per_s": round(self.pinned_copy_peak(), 2),
            }
            res["streaming"]["link_frac_of_pinned_peak"] = round(link / res["streaming"]["pinned_copy_peak_GB_per_s"], 4)
        res["_layers"] = layers
        res["_tokens"] = tokens
        return res

    def pinned_experts(self):
        """Every expert's slice in page-locked host memory (a new pinned tensor)."""
        if getattr(self, "_host", None) is None:
            self._host = self.torch.empty(tuple(self.packed.shape), dtype=self.torch.uint8, pin_memory=True)
            self._host.copy_(self.packed)
        return self._host

    def pinned_copy_peak(self):
        """Host-to-device rate of one 1 GiB copy from page-locked memory."""
        torch = self.torch
        src = self.pinned_experts().view(-1)[:1 << 30]
        dst = torch.empty(1 << 30, dtype=torch.uint8, device=self.dev)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = 0.0
        for _ in range(3):
            ev0.record()
            dst.copy_(src, non_blocking=True)
            ev1.record()
            torch.cuda.synchronize()
            best = max(best, (1 << 30) / (ev0.elapsed_time(ev1) / 1e3) / 1e9)
        del dst
        return best


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", choices=tuple(WORKLOADS), default="decode")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads' summaries")
    ap.add_argument("--cpu-sample", type=int, default=-1,
                    help="oracle decode tokens for cpu_baseline (-1: one per worker process; 0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB elementwise copy first (for scaling --pmc byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.workload)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path (no sharding, no "
              "collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synthetic as S

    torch.cuda.set_device(0)
    b = Bench(S.REAL)
    wl = args.workload
    log(f"{wl}: {args.warmup} warmup + {args.steps} timed steps")
    head = b.run(wl, args.steps, args.warmup, copy_calibration=args.copy_calibration)
    layers, tokens = head.pop("_layers"), head.pop("_tokens")
    extra = {}
    if wl == "decode" and not args.no_extra:
        for other in ("small", "decode_fp4", "prefill", "prefill_fp4", "prefill_mixed", "prefill_hot", "skewed"):
            st = 100 if WORKLOADS[other]["m"] <= 8 else 5 if other == "skewed" else 10
            wu = 3 if other == "skewed" else 20   # the first calls of a workload run slower
            log(f"{other}: {wu} warmup + {st} timed steps")
            r = b.run(other, st, wu)
            r.pop("_layers"), r.pop("_tokens")
            extra[other] = r

    kname, _ = DOMINANT[wl]
    ga = head["gateup_avg_launch_ms"]
    achieved = head["gateup_GB_per_s"]
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": head["config"] + ": dim 5120, inter 2304, 384 routed experts top-6 "
                                         "(Q2_K gate/up, Q3_K down) x q8_1 activations",
            "m": head["m"],
            "layers_in_rotation": head["layers_in_rotation"],
            "token_pool": head["token_pool"],
            "experts_per_step": head["experts_per_step"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("gateup_q8 (routed gate/up + SwiGLU + q8_1 of h; with a bf16 shared expert also "
                       f"{head['shared_rows_in_gateup']} of its down rows)" if head["m"] <= 8
                       else "mmq_gateup_q2k (routed gate/up + SwiGLU)"),
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(wl),
            "bytes_per_launch": head["gateup_bytes_per_launch"],
            "avg_launch_ms": ga,
        },
        "routed_kernels": head["routed_kernels"],
        "all_kernels": head["all_kernels"],
        "layer_GB_per_s": head["layer_expert_GB_per_s"],
        "layer_frac_of_hbm_peak": head["layer_frac_of_hbm_peak"],
        "ms_per_step_with_kernel_events": head["ms_per_step_with_kernel_events"],
        "kernel_timing": "per-kernel start/stop HIP events carried by each launch (hipExtLaunchKernel: the "
                         "kernel's own begin/end timestamps) over a replay of the same steps right after "
                         "the timed region",
        "kernel_avg_ms": head["kernel_avg_ms"],
    }
    result["gateup_routed_only_GB_per_s"] = head["gateup_routed_only_GB_per_s"]
    result["near_ties"] = head["near_ties"]
    for k in ("mmq_i8_mfma_util", "mmq_i8_TOPS", "mmq_frac_of_hbm_peak", "per_call", "graph_replay"):
        if k in head:
            result[k] = head[k]
    if extra:
        result["workloads"] = extra
    if args.cpu_sample != 0 and wl == "decode":
        log("cpu baseline: running the oracle")
        result["cpu_baseline"] = cpu_baseline(layers[0], tokens, b.experts, b.shape,
                                              args.cpu_sample if args.cpu_sample > 0 else None)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
