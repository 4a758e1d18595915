"""GPU backward (moe_backward) against the oracle's float64 gradients: dx,
the three expert weight gradients on every slot, the routing-weight and
logit gradients.

The bar comes from the arithmetic: the per-pair intermediates (w dy, the
SwiGLU output, dG and dU) are rounded once each to the layer's dtype, whose
unit roundoff is 2^-9 (bf16) or 2^-12 (f16), and every gradient element is
a sum of products through at most three of them, so its error is a few unit
roundoffs of the sum's size. Two bars per compared part, FRO = 1e-2 (bf16),
2e-3 (f16), about five unit roundoffs:
  normwise     ||g - ref||_F <= FRO * ||ref||_F;
  elementwise  max |g - ref| <= FRO * max |ref|: one product of rounded
               factors errs by at most ~3 unit roundoffs of its own size,
               which is at most the part's largest value.
The weight gradients are compared slot by slot (every expert slot holding a
kept pair, each against its own norm and largest value, so a wrong light
slot cannot hide under a heavy one; empty slots exactly zero), dx token by
token: a dispatch that runs only the chosen experts must give each slot the
gradient running every expert gives (mini-AGI PR #3, tests/test_dispatch.py).
"""

import numpy as np
import pytest
import torch

import mixture_experts_routed_route_amd as moe
import oracle
import workloads as W
from helpers import gpu_plan, plan_arrays, say, to_dev

pytestmark = pytest.mark.gpu

FRO = {W.BF16: 1e-2, W.F16: 2e-3}


def run_backward(wl, dy, options=None, plan=None):
    p = plan if plan is not None else gpu_plan(wl)
    g = moe.moe_backward(p, wl["x"].cuda(), to_dev(wl["w_gate"]),
                         to_dev(wl["w_up"]), to_dev(wl["w_down"]), dy.cuda(),
                         options=options, want_dtw=True, want_dlogits=True)
    torch.cuda.synchronize()
    return p, {k: v.cpu().numpy().astype(np.float64) for k, v in g.items()}


def close(got, ref, what, dt, quiet=False):
    """Both bars on one part (skipped parts: ref all zero -> got exactly 0)."""
    assert np.all(np.isfinite(got)), what
    if not np.any(ref):
        assert not np.any(got), f"{what}: nonzero where the gradient is zero"
        return 0.0, 0.0
    nref = float(np.linalg.norm(ref))
    nerr = float(np.linalg.norm(got - ref))
    amax = float(np.max(np.abs(ref)))
    emax = float(np.max(np.abs(got - ref)))
    if not quiet:
        say(f"  {what}: |err|_F / |ref|_F = {nerr / nref:.2e}, "
            f"max err / max|ref| = {emax / amax:.2e}")
    assert nerr <= FRO[dt] * nref, f"{what}: {nerr:.3e} > {FRO[dt]} x {nref:.3e}"
    assert emax <= FRO[dt] * amax, f"{what}: max err {emax:.3e} > {FRO[dt]} x {amax:.3e}"
    return nerr / nref, emax / amax


def close_slots(got, ref, experts, counts, what, dt):
    """Each expert slot on its own: the two bars for slots holding kept
    pairs, exact zeros for empty ones."""
    worst = [0.0, 0.0]
    for i, e in enumerate(experts):
        if counts[e] == 0:
            assert not np.any(got[i]), f"{what}[{e}]: empty slot not zero"
            assert not np.any(ref[i])
            continue
        r = close(got[i], ref[i], f"{what}[{e}]", dt, quiet=True)
        worst = [max(worst[0], r[0]), max(worst[1], r[1])]
    say(f"  {what}: {len(experts)} slots, worst |err|_F / |ref|_F = "
        f"{worst[0]:.2e}, worst max err / max|ref| = {worst[1]:.2e}")


def close_rows(got, ref, what, dt):
    """Row by row (tokens); rows whose gradient is zero must be zero."""
    worst = [0.0, 0.0]
    for t in range(ref.shape[0]):
        r = close(got[t], ref[t], f"{what}[{t}]", dt, quiet=True)
        worst = [max(worst[0], r[0]), max(worst[1], r[1])]
    say(f"  {what}: {ref.shape[0]} rows, worst |err|_F / |ref|_F = "
        f"{worst[0]:.2e}, worst max err / max|ref| = {worst[1]:.2e}")


def oracle_grads(wl, p, dy, c, tokens=None, experts=None, want=("dx", "dw", "dtw")):
    a = plan_arrays(p)
    ids = a["topk_id"]
    # the oracle's own route and plan (bit-exact with the GPU's, tested
    # elsewhere) give the weights in float64 and the keep mask
    ids_o, w_o = oracle.route(wl["logits"], wl["k"])
    assert np.array_equal(ids, ids_o)
    pl = oracle.plan(ids_o, wl["E"], wl["capacity_factor"], wl["n_shared"])
    ref = oracle.backward(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids_o,
                          w_o, pl["keep"], dy.numpy().astype(np.float64),
                          E=wl["E"], n_shared=wl["n_shared"],
                          x_dtype=wl["x_dtype"], w_dtype=wl["w_dtype"], c=c,
                          tokens=tokens, experts=experts, want=want)
    if "dtw" in want:
        ref["dlogits"] = oracle.dlogits(ids_o, w_o, ref["dtw"], wl["E"])
    return ref, pl


@pytest.mark.parametrize("dt", [W.BF16, W.F16])
@pytest.mark.parametrize("n_shared,cf,c", [(0, 0.0, 7.0), (1, 1.0, 0.5),
                                           (0, 0.5, 0.0)])
def test_backward_small_all_gradients(dt, n_shared, cf, c):
    wl = W.make_layer(200, 128, 256, 8, 2, dt, seed=61, w_std=0.1,
                      n_shared=n_shared, capacity_factor=cf)
    dy = torch.randn(200, 128, generator=torch.Generator().manual_seed(7))
    say(f"backward small {dt} shared={n_shared} cf={cf} c={c}")
    opts = moe.make_options(swiglu_limit=c)
    p, g = run_backward(wl, dy, opts)
    ref, pl = oracle_grads(wl, p, dy, c)
    counts = plan_arrays(p)["counts"]
    slots = np.arange(wl["E"] + n_shared)
    close(g["dx"], ref["dx"], "dx", dt)
    close_rows(g["dx"], ref["dx"], "dx", dt)
    for key in ("dw_gate", "dw_up", "dw_down"):
        close(g[key], ref[key], key, dt)
        close_slots(g[key], ref[key], slots, counts, key, dt)
    close(g["d_topk_w"], ref["dtw"], "d_topk_w", dt)
    close(g["d_logits"], ref["dlogits"], "d_logits", dt)
    assert np.all(g["d_topk_w"][pl["keep"] == 0] == 0)
    if cf == 0.5:
        assert (pl["keep"] == 0).sum() > 50          # pairs were dropped
    # the logit gradient of a token sums to zero (its weights sum to one)
    assert np.allclose(g["d_logits"].sum(1), 0.0,
                       atol=1e-5 * np.abs(g["d_logits"]).max())


def test_backward_uneven_slots():
    """Slots of very different loads (logit bias: one expert takes nearly
    every token, others a handful of pairs, some none): every slot is
    checked against its own norm and largest value, so an error confined to
    a light slot fails even beside the heavy one."""
    # kept pairs per slot: 300, 81, 42, 20, 1, 2, 0, 1, 0 x 4, 153, 0 x 3,
    # and the shared expert's 300
    bias = torch.tensor([5.0, 2.0, 1.5, 1.0, 0.5, 0.0, -0.5, -1.0, -9.0,
                         -9.0, -9.0, -9.0, 2.5, -9.0, -9.0, -9.0])
    for dt in (W.BF16, W.F16):
        wl = W.make_layer(300, 256, 128, 16, 2, dt, seed=63, w_std=0.1,
                          logit_bias=bias, n_shared=1)
        dy = torch.randn(300, 256, generator=torch.Generator().manual_seed(11))
        say(f"backward uneven slots {dt}")
        p, g = run_backward(wl, dy)
        ref, pl = oracle_grads(wl, p, dy, 7.0)
        counts = plan_arrays(p)["counts"]
        live = counts[:16][counts[:16] > 0]
        assert live.max() > 250 and live.min() <= 3 and (counts == 0).any()
        slots = np.arange(17)
        for key in ("dw_gate", "dw_up", "dw_down"):
            close_slots(g[key], ref[key], slots, counts, key, dt)
        close_rows(g["dx"], ref["dx"], "dx", dt)
        close(g["d_topk_w"], ref["dtw"], "d_topk_w", dt)


@pytest.mark.parametrize("dt", [W.BF16, W.F16])
def test_backward_ragged_tiles(dt):
    """d_model 384 and d_ff 640 (multiples of 128, not of 256): the last
    256-wide block of every product's output is half outside it, and the
    weight gradients' 256-row tiles of D rows end half empty; one expert
    holds more than 256 pairs (two pair tiles, nine 32-pair stages), a
    shared expert every token, and a capacity limit drops pairs."""
    bias = torch.tensor([3.0, 0.5, 0.0, 0.0, -0.5, -1.0, -1.0, -9.0])
    wl = W.make_layer(300, 384, 640, 8, 2, dt, seed=67, w_std=0.08,
                      logit_bias=bias, n_shared=1, capacity_factor=3.5)
    dy = torch.randn(300, 384, generator=torch.Generator().manual_seed(13))
    say(f"backward ragged tiles {dt} D=384 F=640")
    p, g = run_backward(wl, dy)
    ref, pl = oracle_grads(wl, p, dy, 7.0)
    counts = plan_arrays(p)["counts"]
    assert counts[:8].max() > 256 and (pl["keep"] == 0).any()
    slots = np.arange(9)
    for key in ("dw_gate", "dw_up", "dw_down"):
        close(g[key], ref[key], key, dt)
        close_slots(g[key], ref[key], slots, counts, key, dt)
    close_rows(g["dx"], ref["dx"], "dx", dt)
    close(g["d_topk_w"], ref["dtw"], "d_topk_w", dt)
    close(g["d_logits"], ref["dlogits"], "d_logits", dt)


def test_backward_empty_experts_get_zero_gradients():
    # 16 experts, 8 tokens top-1 with logits that favour the first four:
    # most slots hold no pair and must read zero
    bias = torch.tensor([8.0] * 4 + [-8.0] * 12)
    wl = W.make_layer(8, 128, 128, 16, 1, W.BF16, seed=62, logit_bias=bias)
    dy = torch.randn(8, 128, generator=torch.Generator().manual_seed(8))
    dt = W.BF16
    say("backward empty experts")
    p, g = run_backward(wl, dy)
    counts = plan_arrays(p)["counts"]
    empty = np.where(counts == 0)[0]
    assert len(empty) >= 12
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert np.all(g[key][empty] == 0), key
    ref, _ = oracle_grads(wl, p, dy, 7.0)
    close_rows(g["dx"], ref["dx"], "dx", dt)
    for key in ("dw_gate", "dw_up", "dw_down"):
        close_slots(g[key], ref[key], np.arange(16), counts, key, dt)


def test_backward_prefill_sampled():
    """The prefill workload (4096 tokens, d_model 2048, d_ff 768, 128
    experts, top-8, bf16, Zipf popularity): dx of 24 sampled tokens row by
    row; the weight gradients of four slots each on its own: the lightest
    live expert, a middle one, the second heaviest and the heaviest (3974
    pairs)."""
    wl = W.config(3)
    dt = wl["x_dtype"]
    dy = torch.randn(wl["T"], wl["D"], generator=torch.Generator().manual_seed(9))
    say("backward prefill_zipf sampled")
    p, g = run_backward(wl, dy)
    counts = plan_arrays(p)["counts"].astype(np.int64)
    order = np.argsort(counts, kind="stable")
    live = order[counts[order] > 0]
    experts = [int(live[0]), int(live[len(live) // 2]), int(live[-2]),
               int(live[-1])]
    say(f"  slots {experts} holding {[int(counts[e]) for e in experts]} pairs")
    toks = np.unique(np.concatenate([[0, wl["T"] - 1], np.random.default_rng(2).choice(
        wl["T"], 22, replace=False)]))
    ref, _ = oracle_grads(wl, p, dy, 7.0, tokens=toks, experts=experts,
                          want=("dx", "dw"))
    close_rows(g["dx"][toks], ref["dx"], "dx", dt)
    for key in ("dw_gate", "dw_up", "dw_down"):
        close_slots(g[key][experts], ref[key], experts, counts, key, dt)


def test_backward_decode_and_repeat_bitwise():
    wl = W.config(6, T=1)
    dt = wl["x_dtype"]
    dy = torch.randn(1, wl["D"], generator=torch.Generator().manual_seed(10))
    say("backward decode T=1, twice")
    p = gpu_plan(wl)
    _, g1 = run_backward(wl, dy, plan=p)
    _, g2 = run_backward(wl, dy, plan=p)
    for key in g1:
        assert np.array_equal(g1[key], g2[key]), key
    ref, _ = oracle_grads(wl, p, dy, 7.0, want=("dx", "dw", "dtw"))
    counts = plan_arrays(p)["counts"]
    close_rows(g1["dx"], ref["dx"], "dx", dt)
    close(g1["d_topk_w"], ref["dtw"], "d_topk_w", dt)
    for key in ("dw_gate", "dw_up", "dw_down"):
        close_slots(g1[key], ref[key], np.arange(wl["E"] + 1), counts, key, dt)
