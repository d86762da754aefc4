"""CPU checks of the C ABI library: it loads, exports every function that
include/moe.h declares, and its host-only calls behave (no GPU needed)."""
import ctypes
import os
import re

import pytest

import mixture_experts_ffn_gemv_amd as moe
import synthetic as S

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return moe.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 15
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(moe.EXPORTED)


def test_expert_layout_matches_block_sizes(lib):
    for shape in (S.TINY, S.REAL, S.LayerShape(512, 768, 40, 9)):
        cfg = moe.make_cfg(shape.dim, shape.inter, shape.n_routed, shape.topk, max_tokens=4)
        assert moe.moe_expert_layout(cfg) == S.expert_layout(shape)


def test_mxfp4_layout_matches_encoder(lib):
    for shape in (S.TINY, S.REAL, S.LayerShape(512, 768, 40, 9)):
        cfg = moe.make_cfg(shape.dim, shape.inter, shape.n_routed, shape.topk, max_tokens=4,
                           expert_fmt=moe.MOE_EXPERT_MXFP4)
        assert moe.moe_expert_layout(cfg) == S.expert_layout(shape, "fp4")
    bad = moe.make_cfg(256, 256, 16, 2, max_tokens=4, expert_fmt=2)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_expert_layout(bad)
    assert e.value.code == moe.MOE_EINVAL


@pytest.mark.parametrize("bad", [dict(dim=300), dict(dim=0), dict(inter=100), dict(n_routed=0),
                                 dict(topk=0), dict(topk=17), dict(max_tokens=0), dict(gate_temp=0.0),
                                 dict(dim=8448)])
def test_expert_layout_rejects_bad_cfg(lib, bad):
    kw = dict(dim=256, inter=256, n_routed=16, topk=2, gate_temp=1.0, max_tokens=4)
    kw.update(bad)
    cfg = moe.make_cfg(kw["dim"], kw["inter"], kw["n_routed"], kw["topk"], gate_temp=kw["gate_temp"],
                       max_tokens=kw["max_tokens"])
    with pytest.raises(moe.MoeError) as e:
        moe.moe_expert_layout(cfg)
    assert e.value.code == moe.MOE_EINVAL


def test_strerror_and_null_handling(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert moe.strerror(code)
    assert moe.strerror(-99) == "unknown status"
    assert lib.moe_destroy(None) == moe.MOE_OK
    assert lib.moe_create(None, None) == moe.MOE_EINVAL
    assert lib.moe_set_dispatch(None, moe.MOE_DISPATCH_MIXED) == moe.MOE_EINVAL
    assert lib.moe_check(None, None) == moe.MOE_EINVAL
    assert lib.moe_get_stats(None, None) == moe.MOE_EINVAL
    assert lib.moe_quantize_q8_1(None, 1, 32, None, None, None) == moe.MOE_EINVAL
    out = ctypes.c_void_p()
    bad = moe.make_cfg(300, 256, 16, 2)
    assert lib.moe_create(ctypes.byref(bad), ctypes.byref(out)) == moe.MOE_EINVAL
    assert out.value is None


C_TYPES = {"int32_t": ctypes.c_int32, "float": ctypes.c_float, "uint64_t": ctypes.c_uint64,
           "double": ctypes.c_double, "const void*": ctypes.c_void_p, "const float*": ctypes.c_void_p}


def header_struct(name):
    """(type, field) pairs of `typedef struct name { ... } name;` in include/moe.h."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, flags=re.S).group(1)
    return [(" ".join(t.split()), f) for t, f in re.findall(r"([A-Za-z_][\w ]*\*?)\s+(\w+);", body)]


@pytest.mark.parametrize("name", ["moe_cfg", "moe_weights", "moe_stats", "moe_plan"])
def test_binding_structs_match_header(name):
    fields = header_struct(name)
    binding = getattr(moe, name)._fields_
    assert [f for _, f in fields] == [f for f, _ in binding]
    for (ctype, f), (_, pytype) in zip(fields, binding):
        assert ctypes.sizeof(C_TYPES[ctype]) == ctypes.sizeof(pytype), (name, f, ctype)


def test_stats_carry_the_timing_fields_and_near_ties():
    names = [f for _, f in header_struct("moe_stats")]
    for f in ("hits", "misses", "bytes_copied", "route_ms", "fetch_ms", "compute_ms", "near_ties"):
        assert f in names


def test_static_forward_rejects_bad_arguments_before_any_device_call(lib):
    # every check below fails before the library touches a device
    cfg = moe.make_cfg(256, 256, 16, 2)
    w = moe.make_weights(None, None)
    args = lambda c, m, arena=1 << 20: (ctypes.byref(c) if c is not None else None, ctypes.byref(w), arena,
                                         1 << 20, 1 << 20, m, 1 << 20, None, None, None, None)
    assert lib.moe_forward_static(*args(None, 1)) == moe.MOE_EINVAL
    assert lib.moe_forward_static(*args(cfg, 1, arena=None)) == moe.MOE_EINVAL
    for m in (0, 9):
        assert lib.moe_forward_static(*args(cfg, m)) == moe.MOE_EINVAL
    fp4 = moe.make_cfg(256, 256, 16, 2, expert_fmt=moe.MOE_EXPERT_MXFP4)
    assert lib.moe_forward_static(*args(fp4, 1)) == moe.MOE_EINVAL
    assert lib.moe_forward_static(*args(cfg, 1, arena=(1 << 20) + 16)) == moe.MOE_EINVAL   # arena not 256-aligned
