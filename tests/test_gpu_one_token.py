"""One-token calls (T = 1) on bf16 / fp16 layers, and on 4-bit layers with
fp16 x, take the two matrix-vector kernels (gate/up + SwiGLU, then down with the combine) instead of the
split-K tile and the combine kernel. Checked against the oracle: the output,
every pair's unweighted expert output (the pair buffer the combine would
read), and the same call kept on the tile (MOE_OPT_TILED_DECODE), both
within the bar; y in x's dtype is the f32 output rounded once. Shapes: the
short-prompt layer's (D 2048, F 768, top-8 + a shared expert), a capped
plan (the bf16 hi + lo SwiGLU pair) with a binding clamp, k = E, a long F
(the down kernel's K in several passes) and a long D (gate/up in several
passes), an odd number of pairs for the down kernel's groups of four; for
the three 4-bit formats the long-prompt layer's sizes (D 4096, F 2048,
top-8), a capped plan with a shared expert, and long rows for either
product (the pieces of a row in several passes)."""

import numpy as np
import pytest
import torch

import mixture_experts_routed_route_amd as moe
import workloads as W
from helpers import (check_layer, check_pairs, gpu_layer, gpu_layer_views, plan_arrays,
                     say, to_dev)

pytestmark = pytest.mark.gpu

CASES = [
    # dt, D, F, E, k, n_shared, cf, clamp
    (W.BF16, 2048, 768, 128, 8, 1, 0.0, 7.0),
    (W.F16, 2048, 768, 128, 8, 1, 0.0, 7.0),
    (W.BF16, 256, 384, 16, 4, 0, 1.0, 0.5),
    (W.F16, 640, 128, 8, 8, 1, 2.0, 0.0),
    (W.BF16, 128, 4096, 32, 2, 0, 0.0, 7.0),
    (W.F16, 4096, 256, 64, 6, 1, 0.0, 7.0),
    (W.BF16, 384, 1152, 24, 5, 0, 0.0, 7.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-D{c[1]}-F{c[2]}-k{c[4]}")
def test_one_token_against_oracle_and_tile(case):
    dt, D, F, E, k, ns, cf, c = case
    wl = W.make_layer(1, D, F, E, k, dt, seed=D + F + k, n_shared=ns,
                      capacity_factor=cf, swiglu_limit=c, w_std=0.05)
    say(f"one token {case}")
    opts = moe.make_options(swiglu_limit=c)
    p, y, views = gpu_layer_views(wl, options=opts)
    check_layer(wl, y)
    counts = plan_arrays(p)["counts"]
    experts = np.nonzero(counts)[0]
    assert len(experts) == k + ns
    check_pairs(wl, p, views, experts)
    # bf16 carries the low plane exactly when the plan is capped
    assert ("h_lo" in views) == (dt == W.BF16 and cf > 0)
    tiled = moe.make_options(swiglu_limit=c, flags=moe.MOE_OPT_TILED_DECODE)
    _, y_t = gpu_layer(wl, options=tiled, plan=p)
    check_layer(wl, y_t)
    # y in x's dtype: the f32 output rounded once
    x = wl["x"].cuda()
    yx = moe.moe_forward(p, x, wl["w_gate"].cuda(), wl["w_up"].cuda(),
                         wl["w_down"].cuda(), options=opts, y_dtype=x.dtype)
    torch.cuda.synchronize()
    assert torch.equal(yx, y.to(x.dtype))


def test_one_token_phases_and_repeat():
    """The two launches report as phases 3 and 5 (no combine phase), and
    calls repeated on new tokens give the same output as fresh calls."""
    wl = W.config(6, T=1)
    say(f"one token phases {wl['name']}")
    moe.moe_phase_times(reset=True)
    o = moe.make_options(flags=moe.MOE_OPT_PHASE_EVENTS)
    p, y = gpu_layer(wl, options=o)
    ms, calls = moe.moe_phase_times(reset=True)
    assert calls == 1
    assert ms["gateup_thin16"] > 0 and ms["down_thin16"] > 0 and ms["combine"] == 0
    check_layer(wl, y)
    for s in range(3):
        wl2 = W.config(6, T=1, seed=100 + s)
        p2, y2 = gpu_layer(wl2)
        check_layer(wl2, y2)
        _, y3 = gpu_layer(wl2, plan=p2)
        assert torch.equal(y2, y3)


Q4_CASES = [
    # w_dtype, D, F, E, k, n_shared, cf, clamp
    (W.Q4B32, 4096, 2048, 16, 8, 0, 0.0, 7.0),
    (W.Q4A32, 4096, 2048, 16, 8, 0, 0.0, 7.0),
    (W.Q4A64, 4096, 2048, 16, 8, 0, 0.0, 7.0),
    (W.Q4B32, 256, 384, 16, 4, 1, 1.0, 0.5),
    (W.Q4A64, 640, 128, 8, 8, 1, 2.0, 0.0),
    (W.Q4B32, 128, 4096, 32, 2, 0, 0.0, 7.0),
    (W.Q4A32, 8192, 256, 8, 3, 1, 0.0, 7.0),
]


@pytest.mark.parametrize("case", Q4_CASES, ids=lambda c: f"{c[0]}-D{c[1]}-F{c[2]}-k{c[4]}")
def test_one_token_q4_against_oracle_and_tile(case):
    wdt, D, F, E, k, ns, cf, c = case
    wl = W.make_layer(1, D, F, E, k, W.F16, w_dtype=wdt, seed=D + F + k,
                      n_shared=ns, capacity_factor=cf, swiglu_limit=c)
    say(f"one token 4-bit {case}")
    opts = moe.make_options(swiglu_limit=c)
    moe.moe_phase_times(reset=True)
    ph = moe.make_options(swiglu_limit=c, flags=moe.MOE_OPT_PHASE_EVENTS)
    p, y, views = gpu_layer_views(wl, options=ph)
    ms, calls = moe.moe_phase_times(reset=True)
    assert calls == 1 and ms["combine"] == 0   # the down kernel summed y
    check_layer(wl, y)
    counts = plan_arrays(p)["counts"]
    experts = np.nonzero(counts)[0]
    assert len(experts) == k + ns
    check_pairs(wl, p, views, experts)
    tiled = moe.make_options(swiglu_limit=c, flags=moe.MOE_OPT_TILED_DECODE)
    _, y_t = gpu_layer(wl, options=tiled, plan=p)
    check_layer(wl, y_t)
    x = wl["x"].cuda()
    wg, wu, wd = (to_dev(wl[n]) for n in ("w_gate", "w_up", "w_down"))
    yx = moe.moe_forward(p, x, wg, wu, wd, options=opts, y_dtype=x.dtype)
    y2 = moe.moe_forward(p, x, wg, wu, wd, options=opts)
    torch.cuda.synchronize()
    assert torch.equal(yx, y.to(x.dtype))
    assert torch.equal(y2, y)
