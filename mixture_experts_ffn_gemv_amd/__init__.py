"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every function here has the name of the C entry point it calls and forwards
plain pointers and sizes; tensors are torch tensors on the current HIP device
(PyTorch supplies memory and streams, nothing else). Every step of the layer
runs in the HIP kernels of libmoe.so; if the library is not built this module
raises on first use instead of falling back to anything.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_EINVAL = -1
MOE_ENOMEM = -2
MOE_EHIP = -3
MOE_ENONFINITE = -4
MOE_ENOTRESIDENT = -5
MOE_ESTATE = -6
MOE_ESCRATCH = -7

MOE_SHARED_NONE = 0
MOE_SHARED_BF16 = 1
MOE_SHARED_KQUANT = 2

MOE_EXPERT_KQUANT = 0
MOE_EXPERT_MXFP4 = 1

MOE_DISPATCH_MMQ = 0
MOE_DISPATCH_MIXED = 1

MOE_PATH_DECODE = 0
MOE_PATH_GEMV = 1
MOE_PATH_MMQ = 2

MOE_STATIC_SCRATCH_BYTES = 8 << 20

EXPORTED = (
    "moe_create", "moe_destroy", "moe_expert_layout", "moe_pack_expert", "moe_set_slots", "moe_slot_bind",
    "moe_slot_evict",
    "moe_slot_of", "moe_set_host_arena", "moe_route", "moe_forward", "moe_forward_ex", "moe_check",
    "moe_get_stats", "moe_reset_stats", "moe_strerror", "moe_quantize_q8_1", "moe_set_profiling",
    "moe_kernel_times", "moe_set_dispatch", "moe_plan_call", "moe_forward_static",
)

KERNEL_CLASSES = ("router", "quant_h", "topk", "bucket", "gateup", "shared_gateup", "down", "shared_down",
                  "combine")


class moe_cfg(ctypes.Structure):
    _fields_ = [
        ("dim", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("n_routed", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("gate_temp", ctypes.c_float),
        ("norm_topk_prob", ctypes.c_int32),
        ("route_scale", ctypes.c_float),
        ("swiglu_limit", ctypes.c_float),
        ("max_tokens", ctypes.c_int32),
        ("expert_fmt", ctypes.c_int32),
    ]


class moe_weights(ctypes.Structure):
    _fields_ = [
        ("router_w", ctypes.c_void_p),
        ("router_bias", ctypes.c_void_p),
        ("shared_fmt", ctypes.c_int32),
        ("shared_w1", ctypes.c_void_p),
        ("shared_w3", ctypes.c_void_p),
        ("shared_w2", ctypes.c_void_p),
    ]


class moe_stats(ctypes.Structure):
    _fields_ = [
        ("calls", ctypes.c_uint64),
        ("hits", ctypes.c_uint64),
        ("misses", ctypes.c_uint64),
        ("bytes_copied", ctypes.c_uint64),
        ("waves", ctypes.c_uint64),
        ("route_ms", ctypes.c_double),
        ("fetch_ms", ctypes.c_double),
        ("compute_ms", ctypes.c_double),
        ("near_ties", ctypes.c_uint64),
    ]


class moe_plan(ctypes.Structure):
    _fields_ = [
        ("small_routing", ctypes.c_int32),
        ("expert_path", ctypes.c_int32),
        ("shared_rows_router", ctypes.c_int32),
        ("shared_rows_topk", ctypes.c_int32),
        ("shared_rows_gateup", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code})")


_lib = None


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        sigs = {
            "moe_create": [P(moe_cfg), P(vp)],
            "moe_destroy": [vp],
            "moe_expert_layout": [P(moe_cfg), P(sz), P(sz), P(sz), P(sz)],
            "moe_pack_expert": [P(moe_cfg), vp, vp, vp],
            "moe_set_slots": [vp, vp, i32],
            "moe_slot_bind": [vp, i32, i32],
            "moe_slot_evict": [vp, i32],
            "moe_slot_of": [vp, i32, P(i32)],
            "moe_set_host_arena": [vp, vp, sz],
            "moe_route": [vp, P(moe_weights), vp, i32, vp, vp, vp],
            "moe_forward": [vp, P(moe_weights), vp, i32, vp, vp],
            "moe_forward_ex": [vp, P(moe_weights), vp, i32, vp, vp, vp, vp],
            "moe_check": [vp, vp],
            "moe_get_stats": [vp, P(moe_stats)],
            "moe_reset_stats": [vp],
            "moe_quantize_q8_1": [vp, i32, i32, vp, vp, vp],
            "moe_set_profiling": [vp, i32],
            "moe_set_dispatch": [vp, i32],
            "moe_kernel_times": [vp, P(ctypes.c_double), P(ctypes.c_int64), i32],
            "moe_plan_call": [vp, i32, i32, P(moe_plan)],
            "moe_forward_static": [P(moe_cfg), P(moe_weights), vp, vp, vp, i32, vp, vp, vp, vp, vp],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code):
    return lib().moe_strerror(code).decode()


def _check(rc, where):
    if rc != MOE_OK:
        raise MoeError(rc, where)
    return rc


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def make_cfg(dim, inter, n_routed, topk, gate_temp=1.0, norm_topk_prob=True, route_scale=1.5,
             swiglu_limit=10.0, max_tokens=1, expert_fmt=MOE_EXPERT_KQUANT):
    return moe_cfg(dim, inter, n_routed, topk, gate_temp, int(bool(norm_topk_prob)), route_scale,
                   swiglu_limit, max_tokens, expert_fmt)


def make_weights(router_w, router_bias, shared_fmt=MOE_SHARED_NONE, shared_w1=None, shared_w3=None,
                 shared_w2=None):
    return moe_weights(_ptr(router_w), _ptr(router_bias), shared_fmt, _ptr(shared_w1), _ptr(shared_w3),
                       _ptr(shared_w2))


# ----------------------------------------------------------------------------- entry points

def moe_create(cfg):
    ctx = ctypes.c_void_p()
    _check(lib().moe_create(ctypes.byref(cfg), ctypes.byref(ctx)), "moe_create")
    return ctx


def moe_destroy(ctx):
    return _check(lib().moe_destroy(ctx), "moe_destroy")


def moe_expert_layout(cfg):
    """-> (slot_bytes, off_w1, off_w3, off_w2)"""
    out = [ctypes.c_size_t() for _ in range(4)]
    _check(lib().moe_expert_layout(ctypes.byref(cfg), *[ctypes.byref(o) for o in out]), "moe_expert_layout")
    return tuple(o.value for o in out)


def moe_pack_expert(cfg, src, dst, stream=None):
    return _check(lib().moe_pack_expert(ctypes.byref(cfg), _ptr(src), _ptr(dst), _stream(stream)), "moe_pack_expert")


def pack_experts(cfg, arena, stream=None):
    """Expert slices in plain GGUF row order, uint8 [n, slot_bytes] on the
    device -> a new tensor of the same shape in the slot layout."""
    out = torch.empty_like(arena)
    for e in range(arena.shape[0]):
        moe_pack_expert(cfg, arena[e], out[e], stream)
    return out


def moe_set_slots(ctx, arena, n_slots):
    return _check(lib().moe_set_slots(ctx, _ptr(arena), n_slots), "moe_set_slots")


def moe_slot_bind(ctx, expert, slot):
    return _check(lib().moe_slot_bind(ctx, expert, slot), "moe_slot_bind")


def moe_slot_evict(ctx, expert):
    return _check(lib().moe_slot_evict(ctx, expert), "moe_slot_evict")


def moe_slot_of(ctx, expert):
    s = ctypes.c_int32()
    _check(lib().moe_slot_of(ctx, expert, ctypes.byref(s)), "moe_slot_of")
    return s.value


def moe_set_host_arena(ctx, pinned, stride):
    return _check(lib().moe_set_host_arena(ctx, _ptr(pinned), stride), "moe_set_host_arena")


def moe_route(ctx, w, x, m, weights_out, idx_out, stream=None):
    return _check(lib().moe_route(ctx, ctypes.byref(w), _ptr(x), m, _ptr(weights_out), _ptr(idx_out),
                                  _stream(stream)), "moe_route")


def moe_forward(ctx, w, x, m, out, stream=None):
    return _check(lib().moe_forward(ctx, ctypes.byref(w), _ptr(x), m, _ptr(out), _stream(stream)), "moe_forward")


def moe_forward_ex(ctx, w, x, m, out, weights_out=None, idx_out=None, stream=None):
    return _check(lib().moe_forward_ex(ctx, ctypes.byref(w), _ptr(x), m, _ptr(out), _ptr(weights_out),
                                       _ptr(idx_out), _stream(stream)), "moe_forward_ex")


def moe_plan_call(ctx, m, shared_fmt):
    """-> dict of the moe_plan fields for a call of m tokens."""
    p = moe_plan()
    _check(lib().moe_plan_call(ctx, m, shared_fmt, ctypes.byref(p)), "moe_plan_call")
    return {f: getattr(p, f) for f, _ in moe_plan._fields_}


def moe_forward_static(cfg, w, arena, slot_table, x, m, out, weights_out=None, idx_out=None, status=None,
                       stream=None):
    return _check(lib().moe_forward_static(ctypes.byref(cfg), ctypes.byref(w), _ptr(arena), _ptr(slot_table),
                                           _ptr(x), m, _ptr(out), _ptr(weights_out), _ptr(idx_out), _ptr(status),
                                           _stream(stream)), "moe_forward_static")


def moe_quantize_q8_1(x, rows, cols, q_out, d_out, stream=None):
    return _check(lib().moe_quantize_q8_1(_ptr(x), rows, cols, _ptr(q_out), _ptr(d_out), _stream(stream)),
                  "moe_quantize_q8_1")


def moe_check(ctx, stream=None):
    """Synchronise and return the device status code (does not raise)."""
    return lib().moe_check(ctx, _stream(stream))


def moe_set_dispatch(ctx, mode):
    """MOE_DISPATCH_MMQ (the default) or MOE_DISPATCH_MIXED (GEMVs for groups of <= 8 rows, MMQ above)."""
    return _check(lib().moe_set_dispatch(ctx, int(mode)), "moe_set_dispatch")


def moe_set_profiling(ctx, on):
    return _check(lib().moe_set_profiling(ctx, int(bool(on))), "moe_set_profiling")


def moe_kernel_times(ctx):
    """-> {kernel class: (summed ms, launches)} since profiling was switched on or last read."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().moe_kernel_times(ctx, ms, cnt, n), "moe_kernel_times")
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_CLASSES)}


def moe_get_stats(ctx):
    s = moe_stats()
    _check(lib().moe_get_stats(ctx, ctypes.byref(s)), "moe_get_stats")
    return {f: getattr(s, f) for f, _ in moe_stats._fields_}


def moe_reset_stats(ctx):
    return _check(lib().moe_reset_stats(ctx), "moe_reset_stats")
