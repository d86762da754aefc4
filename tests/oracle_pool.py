"""The float64 oracle on many rows of a real-shape layer, in several processes.

The oracle decodes every expert a row picks (about two seconds per real-shape
expert), so checking tens of sampled rows one process at a time takes minutes.
Here the rows are dealt out to worker processes, each running the oracle's
own moe_layer on its share; the rows' results are put back in order. The
workers import numpy and the oracle only (started fresh, not forked), and
receive the bytes of the experts their rows pick.
"""
import concurrent.futures
import multiprocessing
import os

import numpy as np

MAX_WORKERS = 16   # the host share of one GPU


def _run(args):
    import oracle
    cfg_args, cfg_kw, x_bits, wr_bits, bias, experts, shared = args
    cfg = oracle.MoeCfg(*cfg_args, **cfg_kw)
    r = oracle.moe_layer(cfg, x_bits, wr_bits, bias, lambda e: experts[e], shared)
    return r["y"], r["idx"]


def workers_for(n_rows):
    return max(1, min(MAX_WORKERS, os.cpu_count() or 1, n_rows))


def oracle_rows(cfg_args, cfg_kw, x_bits, wr_bits, bias, expert_bytes, shared, picks, workers=None):
    """moe_layer's y and idx for the rows of x_bits, computed in parallel.

    cfg_args / cfg_kw: oracle.MoeCfg arguments; expert_bytes(e) -> uint8 slice
    of expert e; picks: the rows' picked experts [rows, k] (from the oracle's
    routing), used only to hand each worker the experts it needs."""
    n = x_bits.shape[0]
    w = workers or workers_for(n)
    shares = [list(range(i, n, w)) for i in range(w)]
    cache = {}
    tasks = []
    for rows in shares:
        need = sorted(set(int(e) for e in np.asarray(picks)[rows].reshape(-1)))
        for e in need:
            if e not in cache:
                cache[e] = expert_bytes(e)
        tasks.append((cfg_args, cfg_kw, x_bits[rows], wr_bits, bias, {e: cache[e] for e in need}, shared))
    if w == 1:
        results = [_run(tasks[0])]
    else:
        ctx = multiprocessing.get_context("spawn")
        with concurrent.futures.ProcessPoolExecutor(max_workers=w, mp_context=ctx) as pool:
            results = list(pool.map(_run, tasks))
    y = np.zeros((n,) + results[0][0].shape[1:])
    idx = np.zeros((n,) + results[0][1].shape[1:], dtype=results[0][1].dtype)
    for rows, (yr, ir) in zip(shares, results):
        y[rows] = yr
        idx[rows] = ir
    return {"y": y, "idx": idx}
