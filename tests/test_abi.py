"""
The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments on the host before any
launch. Without a device, a valid call reports MOE_EHIP with a message.
"""

import ctypes
import glob
import os
import re

import pytest
import torch

import mixture_experts_routed_route_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return moe.library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert "moe_forward" in names and "moe_plan_create" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTED)
    assert "gfx950" in moe.moe_version()


def test_options_default(lib):
    o = moe.moe_options_default()
    assert o.swiglu_limit == 7.0
    assert o.fat_rows == 64
    assert o.splitk_max_pairs > 0
    assert o.flags == 0


def _desc(T=64, E=8, k=2, n_shared=0, cf=0.0):
    return moe.PlanDesc(T, E, k, n_shared, cf)


@pytest.mark.parametrize("kw", [
    dict(k=0), dict(k=9), dict(E=0), dict(E=1025, k=1), dict(T=-1),
    dict(n_shared=2), dict(cf=-1.0), dict(cf=float("nan")),
    dict(cf=float("inf")), dict(T=1 << 30, k=2),
])
def test_plan_desc_validation(lib, kw):
    d = _desc(**kw)
    assert lib.moe_plan_workspace_bytes(ctypes.byref(d)) == 0
    h = ctypes.c_void_p()
    st = lib.moe_plan_create(ctypes.byref(d), 0x1000, 0x10000, 1 << 20, None,
                             ctypes.byref(h))
    assert st == moe.MOE_EINVAL
    assert moe.moe_last_error()
    assert not h.value


def test_plan_pointer_and_workspace_validation(lib):
    d = _desc()
    need = lib.moe_plan_workspace_bytes(ctypes.byref(d))
    assert need > 0
    h = ctypes.c_void_p()
    assert lib.moe_plan_create(ctypes.byref(d), None, 0x10000, need, None,
                               ctypes.byref(h)) == moe.MOE_EINVAL
    assert lib.moe_plan_create(ctypes.byref(d), 0x1000, None, need, None,
                               ctypes.byref(h)) == moe.MOE_EINVAL
    assert lib.moe_plan_create(ctypes.byref(d), 0x1004, 0x10000, need, None,
                               ctypes.byref(h)) == moe.MOE_EINVAL   # misaligned
    assert lib.moe_plan_create(ctypes.byref(d), 0x1000, 0x10010, need, None,
                               ctypes.byref(h)) == moe.MOE_EINVAL   # ws align
    assert lib.moe_plan_create(ctypes.byref(d), 0x1000, 0x10000, need - 1,
                               None, ctypes.byref(h)) == moe.MOE_EWORKSPACE
    assert "workspace" in moe.moe_last_error()
    assert lib.moe_plan_create(ctypes.byref(d), 0x1000, 0x10000, need, None,
                               None) == moe.MOE_EINVAL


def test_workspace_grows_with_tokens(lib):
    a = lib.moe_plan_workspace_bytes(ctypes.byref(_desc(T=64)))
    b = lib.moe_plan_workspace_bytes(ctypes.byref(_desc(T=640)))
    c = lib.moe_plan_workspace_bytes(ctypes.byref(_desc(T=640, n_shared=1)))
    assert 0 < a < b < c
    assert a % 256 == 0


def test_forward_needs_a_plan(lib):
    w = moe.Weight(moe.MOE_BF16, 0x1000, None)
    st = lib.moe_forward(None, 0x1000, moe.MOE_BF16, w, w, w, 128, 128,
                         0x2000, moe.MOE_F32, 0x10000, 1 << 20, None, None)
    assert st == moe.MOE_EINVAL
    assert lib.moe_forward_workspace_bytes(None, 128, 128, moe.MOE_BF16,
                                           moe.MOE_BF16, None) == 0


def test_dequant_validation(lib):
    assert lib.moe_dequant_q4(0x1000, 0x2000, 4, 48, 0x3000, None) == moe.MOE_EINVAL
    assert lib.moe_dequant_q4(0x1000, 0x2000, -1, 64, 0x3000, None) == moe.MOE_EINVAL
    assert lib.moe_dequant_q4(None, None, 0, 64, None, None) == moe.MOE_OK
    assert lib.moe_dequant_q4(0x1008, 0x2000, 4, 64, 0x3000, None) == moe.MOE_EINVAL


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="checks the no-device error path")
def test_no_device_reports_ehip(lib):
    d = _desc()
    need = lib.moe_plan_workspace_bytes(ctypes.byref(d))
    h = ctypes.c_void_p()
    st = lib.moe_plan_create(ctypes.byref(d), 0x1000, 0x10000, need, None,
                             ctypes.byref(h))
    assert st == moe.MOE_EHIP
    assert "hip" in moe.moe_last_error().lower()
    assert not h.value
    ms, calls = moe.moe_phase_times()
    assert calls == 0 and all(v == 0 for v in ms.values())


def test_python_binding_rejects_bad_tensors():
    with pytest.raises(ValueError):
        moe.moe_plan_create(torch.zeros(4, 4, dtype=torch.float64), 2)
    with pytest.raises(ValueError):
        moe.moe_dequant_q4(torch.zeros(4, 16, dtype=torch.int8),
                           torch.zeros(4, 1, dtype=torch.float16))


def _route(lib, d, x=0x1000, xdt=None, w=0x2000, D=128, zw=1e-3,
           logits=0x3000, stats=0x4000, want=None, ws=0x10000,
           nbytes=1 << 20, out=True):
    h = ctypes.c_void_p()
    return lib.moe_route(ctypes.byref(d), x,
                         moe.MOE_BF16 if xdt is None else xdt, w, D, zw,
                         logits, stats, want, ws, nbytes, 0, None,
                         ctypes.byref(h) if out else None), h


def test_route_validation(lib):
    d = _desc()
    need = lib.moe_route_workspace_bytes(ctypes.byref(d), 128)
    assert need > lib.moe_plan_workspace_bytes(ctypes.byref(d)) and need % 256 == 0
    assert lib.moe_route_workspace_bytes(ctypes.byref(d), 12) == 0      # D % 8
    assert lib.moe_route_workspace_bytes(ctypes.byref(_desc(k=0)), 128) == 0
    bad = [dict(xdt=moe.MOE_Q4B32), dict(D=0), dict(D=100), dict(zw=float("nan")),
           dict(zw=float("inf")), dict(x=None), dict(w=None), dict(logits=None),
           dict(x=0x1004), dict(logits=0x3008), dict(stats=0x4004),
           dict(want=0x5002), dict(ws=None), dict(ws=0x10010), dict(out=False)]
    for kw in bad:
        st, h = _route(lib, d, nbytes=need, **kw)
        want = moe.MOE_EUNSUPPORTED if "xdt" in kw else moe.MOE_EINVAL
        assert st == want, kw
        assert not h.value
    st, _ = _route(lib, d, nbytes=need - 1)
    assert st == moe.MOE_EWORKSPACE
    st, _ = _route(lib, _desc(E=0), nbytes=need)
    assert st == moe.MOE_EINVAL


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="checks the no-device error path")
def test_route_no_device_reports_ehip(lib):
    d = _desc()
    need = lib.moe_route_workspace_bytes(ctypes.byref(d), 128)
    st, h = _route(lib, d, nbytes=need)
    assert st == moe.MOE_EHIP and not h.value


def test_python_route_rejects_bad_tensors():
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_route(x, torch.zeros(8, 16, dtype=torch.float16), 2)
    with pytest.raises(ValueError):
        moe.moe_route(x, torch.zeros(8, 12, dtype=torch.bfloat16), 2)
    with pytest.raises(ValueError):
        moe.moe_route(x.view(-1), torch.zeros(8, 16, dtype=torch.bfloat16), 2)


def test_affine_params_shape_picks_format():
    d = torch.zeros(2, 8, 64, dtype=torch.uint8)
    assert moe.q4_dtype(d, torch.zeros(2, 8, 4, dtype=torch.float16)) == moe.MOE_Q4B32
    assert moe.q4_dtype(d, torch.zeros(2, 8, 4, 2, dtype=torch.float16)) == moe.MOE_Q4A32
    assert moe.q4_dtype(d, torch.zeros(2, 8, 2, 2, dtype=torch.float16)) == moe.MOE_Q4A64
    with pytest.raises(ValueError):
        moe.q4_dtype(d, torch.zeros(2, 8, 3, 2, dtype=torch.float16))


def test_backward_validation(lib):
    assert lib.moe_backward_workspace_bytes(None, 128, 128, moe.MOE_BF16) == 0
    w = moe.Weight(moe.MOE_BF16, 0x1000, None)
    st = lib.moe_backward(None, 0x1000, moe.MOE_BF16, w, w, w, 128, 128, 0x2000,
                          0x3000, 0x4000, 0x5000, 0x6000, None, None, 0x10000,
                          1 << 20, None, None)
    assert st == moe.MOE_EINVAL


class _FakePlan:
    """Just the shape of a plan: the binding's checks run before any call."""
    def __init__(self, T, E, k, n_shared=0):
        self.T, self.E, self.k, self.n_shared = T, E, k, n_shared
        self.handle = None


@pytest.mark.parametrize("case", ["gate_experts", "up_shape", "down_shape",
                                  "shared_missing", "mixed_dtype", "q4_data",
                                  "q4_params", "q4_mixed_format"])
def test_python_weight_shapes_rejected_before_launch(case):
    T, D, F, E = 4, 128, 256, 8
    bf = dict(dtype=torch.bfloat16)
    x = torch.zeros(T, D, **bf)
    wg, wu, wd = (torch.zeros(E, F, D, **bf), torch.zeros(E, F, D, **bf),
                  torch.zeros(E, D, F, **bf))
    plan = _FakePlan(T, E, 2)
    if case == "gate_experts":
        wg = torch.zeros(E - 1, F, D, **bf)
    elif case == "up_shape":
        wu = torch.zeros(E, F, D + 128, **bf)
    elif case == "down_shape":
        wd = torch.zeros(E, F, D, **bf)
    elif case == "shared_missing":
        plan = _FakePlan(T, E, 2, n_shared=1)
    elif case == "mixed_dtype":
        wu = torch.zeros(E, F, D, dtype=torch.float16)
    else:
        x = torch.zeros(T, D, dtype=torch.float16)
        def q4(N, K, G=None):
            d = torch.zeros(E, N, K // 2, dtype=torch.uint8)
            p = (torch.zeros(E, N, K // 32, dtype=torch.float16) if G is None
                 else torch.zeros(E, N, K // G, 2, dtype=torch.float16))
            return d, p
        wg, wu, wd = q4(F, D), q4(F, D), q4(D, F)
        if case == "q4_data":
            wd = (torch.zeros(E, D, F, dtype=torch.uint8), wd[1])
        elif case == "q4_params":
            wu = (wu[0], torch.zeros(E, F - 1, D // 32, dtype=torch.float16))
        else:
            wd = q4(D, F, 64)
    with pytest.raises(ValueError):
        moe.moe_forward(plan, x, wg, wu, wd)
    if case in ("gate_experts", "up_shape", "down_shape", "shared_missing"):
        with pytest.raises(ValueError):
            moe.moe_backward(plan, x, wg, wu, wd, torch.zeros(T, D))


def test_binding_constants_match_the_header():
    """The binding's option flags, phase count and status codes are the
    header's #defines (read from include/moe.h), and MOE_OPT_PHASE_ONLY(p)
    is the header's macro for every phase, as a signed 32-bit flags value."""
    import os
    import re

    import mixture_experts_routed_route_amd as moe

    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "moe.h")).read()
    defs = dict(re.findall(r"#define\s+(MOE_\w+)\s+\(?(-?\d+)\)?\s*$", hdr, re.M))
    for name in ("MOE_OPT_PHASE_EVENTS", "MOE_OPT_BF16_PLAIN_H", "MOE_OPT_EXACT_ROUTES",
                 "MOE_OPT_BF16_SPLIT_H", "MOE_OPT_ONE_STREAM", "MOE_OPT_TILED_DECODE",
                 "MOE_OPT_PHASE_SHIFT",
                 "MOE_N_PHASES"):
        assert name in defs, name
        assert getattr(moe, name) == int(defs[name]), name
    assert len(moe.PHASES) == moe.MOE_N_PHASES
    for p in range(moe.MOE_N_PHASES):
        v = (1 << (int(defs["MOE_OPT_PHASE_SHIFT"]) + p)) & 0xFFFFFFFF
        v = v - (1 << 32) if v >= (1 << 31) else v
        assert moe.MOE_OPT_PHASE_ONLY(p) == v
