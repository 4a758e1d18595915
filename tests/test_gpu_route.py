"""GPU router (moe_route) against the oracle: logits = x . w_router^T within
an fp32-accumulation bound, the plan over those logits bit-exact, and the
routing statistics (top-k mass, wanted experts, z-loss, balance term, aux)
against the oracle's double-precision values computed from the same logits.

Where floating point decides an integer (a token's wanted count), the GPU
decides in fp32; a token whose double-precision running mass lies within
1e-5 of 0.9 at the crossing may differ by one, every other token matches.
"""

import numpy as np
import pytest
import torch

import mixture_experts_routed_route_amd as moe
import oracle
import workloads as W
from helpers import check_plan, plan_arrays, say

pytestmark = pytest.mark.gpu

# |l - ref| <= LOGIT_TOL * sum_d |x_d w_d|: fp32 sums of exact products over
# at most 2^20 terms in blocks stay far inside this; a dropped or doubled
# term of average size (1 / D of the bound's sum) does not.
LOGIT_TOL = 2e-5
STAT_RTOL = 1e-5
WANT_AMBIG = 1e-5


def run_route(wl, z_weight=1e-3):
    x = wl["x"].cuda()
    w = wl["w_router"].cuda()
    plan, logits, stats, want = moe.moe_route(
        x, w, wl["k"], wl["capacity_factor"], wl["n_shared"],
        z_weight=z_weight, want_per_token=True)
    torch.cuda.synchronize()
    return plan, logits.cpu(), stats.cpu().numpy(), want.cpu().numpy()


def check_logits(wl, logits, rows=None):
    x, w = wl["x"], wl["w_router"]
    if rows is not None:
        x = x[torch.as_tensor(rows)]
    ref = oracle.router_logits(x, w, wl["dtype"])
    bound = oracle.router_logits(x.abs(), w.abs(), wl["dtype"])
    got = logits.numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
    err = np.abs(got - ref)
    assert np.all(err <= LOGIT_TOL * bound + 1e-30), float((err / (bound + 1e-30)).max())
    return ref


def ambiguous_tokens(logits):
    """Tokens whose double-precision running mass is within WANT_AMBIG of 0.9
    at the crossing count or the one before it."""
    lg = logits.numpy().astype(np.float64)
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    run = np.cumsum(-np.sort(-p, axis=1), axis=1)
    m = np.argmax(run >= 0.9, axis=1)                 # 0-based crossing
    at = run[np.arange(len(m)), m]
    before = np.where(m > 0, run[np.arange(len(m)), np.maximum(m - 1, 0)], 0.0)
    return (np.abs(at - 0.9) <= WANT_AMBIG) | (np.abs(before - 0.9) <= WANT_AMBIG)


def check_stats(wl, logits, stats, want, z_weight=1e-3):
    ref, want_ref = oracle.router_stats(logits.numpy(), wl["k"], z_weight)
    amb = ambiguous_tokens(logits)
    diff = want.astype(np.int64) - want_ref
    assert np.all(diff[~amb] == 0), f"{int((diff[~amb] != 0).sum())} tokens differ"
    assert np.all(np.abs(diff[amb]) <= 1)
    T = len(want)
    for i, key in enumerate(oracle.ROUTER_STATS):
        if key == "want_k":
            assert stats[i] == pytest.approx(want.mean() if T else 0.0, rel=1e-6)
            continue
        assert stats[i] == pytest.approx(ref[key], rel=STAT_RTOL, abs=1e-30), key
    assert np.all(stats[5:] == 0)
    return ref


CASES = [
    # (T, D, E, k, dtype, cf): fp32 dot, bf16 64x64 tiles, ragged shapes
    (64, 128, 8, 2, "f32", 0.0),
    (2048, 512, 128, 2, "bf16", 1.5),
    (4096, 2048, 128, 8, "bf16", 0.0),
    (1, 4096, 256, 8, "f16", 0.0),
    (7, 256, 64, 4, "bf16", 0.0),
    (64, 1024, 128, 8, "f16", 0.0),
    (65, 1024, 128, 8, "f16", 0.0),
    (200, 768, 1000, 16, "bf16", 3.0),
    (300, 512, 999, 3, "f16", 0.0),
    (130, 40, 3, 1, "bf16", 0.0),
    (90, 8, 1, 1, "f16", 0.0),
    (333, 96, 513, 9, "f32", 0.0),
    # 128 x 128 tiles (at least 128 of them), ragged in tokens and experts
    (8200, 256, 256, 8, "bf16", 0.0),
    (5500, 128, 300, 4, "f16", 1.5),
]


@pytest.mark.parametrize("T,D,E,k,dt,cf", CASES)
def test_route_against_oracle(T, D, E, k, dt, cf):
    wl = W.make_router(T, D, E, k, dt, seed=T + E, capacity_factor=cf,
                       spread=0.7)
    say(f"route T={T} D={D} E={E} k={k} {dt} cf={cf}")
    plan, logits, stats, want = run_route(wl)
    check_logits(wl, logits)
    wl_plan = dict(logits=logits, k=k, E=E, capacity_factor=cf, n_shared=0)
    check_plan(wl_plan, plan)
    check_stats(wl, logits, stats, want)


def test_route_long_prompt_sampled():
    """The 13,312-token, 4096-wide, 256-expert fp16 router (128 x 128 tiles):
    logits of 512 sampled tokens plus the first and last, the whole plan and
    the statistics over all tokens."""
    wl = W.make_router(13312, 4096, 256, 8, "f16", seed=4, spread=0.5)
    say("route long prompt 13312 x 4096 -> 256")
    plan, logits, stats, want = run_route(wl)
    rows = np.unique(np.concatenate([[0, 13311], np.random.default_rng(1).choice(
        13312, 512, replace=False)]))
    check_logits(wl, logits, rows)
    check_plan(dict(logits=logits, k=8, E=256, capacity_factor=0.0,
                    n_shared=0), plan)
    check_stats(wl, logits, stats, want)


def test_route_plan_equals_plan_create_and_repeats_bitwise():
    wl = W.make_router(3000, 1024, 128, 8, "bf16", seed=9, spread=1.0)
    x, w = wl["x"].cuda(), wl["w_router"].cuda()
    say("route determinism 3000 x 1024 -> 128")
    p1, l1, s1 = moe.moe_route(x, w, 8, 1.5)
    p2, l2, s2 = moe.moe_route(x, w, 8, 1.5)
    p3 = moe.moe_plan_create(l1, 8, 1.5)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(s1, s2)
    a, b, c = plan_arrays(p1), plan_arrays(p2), plan_arrays(p3)
    for key in a:
        assert np.array_equal(a[key], b[key]) and np.array_equal(a[key], c[key]), key


def test_route_z_weight_and_no_statistics():
    wl = W.make_router(500, 256, 64, 4, "f16", seed=2)
    x, w = wl["x"].cuda(), wl["w_router"].cuda()
    say("route z_weight")
    _, l0, s0 = moe.moe_route(x, w, 4, z_weight=0.0)
    _, l1, s1 = moe.moe_route(x, w, 4, z_weight=0.25)
    torch.cuda.synchronize()
    s0, s1 = s0.cpu().numpy(), s1.cpu().numpy()
    assert np.array_equal(s0[:4], s1[:4])
    assert s0[4] == s0[3]
    assert s1[4] == pytest.approx(s1[3] + 0.25 * s1[2], rel=1e-6)
    # statistics off: the C call with NULL stats and want still routes
    import ctypes
    L = moe.library()
    d = moe.PlanDesc(500, 64, 4, 0, 0.0)
    nb = L.moe_route_workspace_bytes(ctypes.byref(d), 256)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    lg = torch.empty(500, 64, dtype=torch.float32, device="cuda")
    h = ctypes.c_void_p()
    assert L.moe_route(ctypes.byref(d), x.data_ptr(), moe.MOE_F16, w.data_ptr(),
                       256, ctypes.c_float(0.0), lg.data_ptr(), None, None,
                       ws.data_ptr(), nb, 0, moe._stream(x.device),
                       ctypes.byref(h)) == moe.MOE_OK
    torch.cuda.synchronize()
    assert torch.equal(lg, l0)
    L.moe_plan_destroy(h)


def test_route_empty_prompt():
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(16, 64, dtype=torch.bfloat16, device="cuda")
    say("route T=0")
    plan, logits, stats, want = moe.moe_route(x, w, 2, want_per_token=True)
    torch.cuda.synchronize()
    assert logits.shape == (0, 16) and want.numel() == 0
    assert torch.all(stats.cpu() == 0)
    assert moe.moe_plan_stats_get(plan)["kept"] == 0


def test_route_nan_input_row():
    wl = W.make_router(100, 128, 32, 2, "f16", seed=5)
    x = wl["x"].clone()
    x[17, 3] = float("nan")
    say("route NaN row")
    plan, logits, stats = moe.moe_route(x.cuda(), wl["w_router"].cuda(), 2)
    torch.cuda.synchronize()
    lg = logits.cpu()
    assert torch.isnan(lg[17]).all() and torch.isfinite(lg[:17]).all()
    assert moe.moe_plan_stats_get(plan)["nonfinite"] == 32
    assert np.isnan(stats.cpu().numpy()[2])   # the z-loss sees the NaN row
