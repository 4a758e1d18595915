"""GPU backward (moe_backward) against the oracle's float64 gradients: dx,
the three expert weight gradients on every slot, the routing-weight and
logit gradients.

The bar comes from the arithmetic: the per-pair intermediates (w dy, the
SwiGLU output, dG and dU) are rounded once each to the layer's dtype, whose
unit roundoff is 2^-9 (bf16) or 2^-12 (f16), and every gradient element is
a sum of products through at most three of them, so its error is a few unit
roundoffs of the sum's size. Per gradient tensor (the compared part):
||g - ref||_F <= FRO[dt] * ||ref||_F, FRO = 1e-2 (bf16), 2e-3 (f16),
about five unit roundoffs."""

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


def close(got, ref, what, dt):
    assert np.all(np.isfinite(got)), what
    nref = float(np.linalg.norm(ref))
    nerr = float(np.linalg.norm(got - ref))
    rms = nref / np.sqrt(max(ref.size, 1))
    say(f"  {what}: |err|_F / |ref|_F = {nerr / (nref + 1e-300):.2e}, "
        f"max err / RMS = {float(np.max(np.abs(got - ref))) / (rms + 1e-300):.2e}")
    assert nerr <= FRO[dt] * nref + 1e-30, f"{what}: {nerr:.3e} > {FRO[dt]} x {nref:.3e}"


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
    close(g["dx"], ref["dx"], "dx", dt)
    close(g["dw_gate"], ref["dw_gate"], "dw_gate", dt)
    close(g["dw_up"], ref["dw_up"], "dw_up", dt)
    close(g["dw_down"], ref["dw_down"], "dw_down", dt)
    close(g["d_topk_w"], ref["dtw"], "d_topk_w", dt)
    close(g["d_logits"], ref["dlogits"], "d_logits", dt)
    assert np.all(g["d_topk_w"][pl["keep"] == 0] == 0)
    if cf == 0.5:
        assert (pl["keep"] == 0).sum() > 50          # pairs were dropped
    # the logit gradient of a token sums to zero (its weights sum to one)
    assert np.allclose(g["d_logits"].sum(1), 0.0,
                       atol=1e-5 * np.abs(g["d_logits"]).max())


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
    close(g["dx"], ref["dx"], "dx", dt)
    close(g["dw_down"], ref["dw_down"], "dw_down", dt)


def test_backward_prefill_sampled():
    """The prefill workload (4096 tokens, d_model 2048, d_ff 768, 128
    experts, top-8, bf16, Zipf popularity): dx of 24 sampled tokens, the
    weight gradients of three experts (the lightest, a middle and a heavier
    one), the routing-weight gradients of every token."""
    wl = W.config(3)
    dt = wl["x_dtype"]
    dy = torch.randn(wl["T"], wl["D"], generator=torch.Generator().manual_seed(9))
    say("backward prefill_zipf sampled")
    p, g = run_backward(wl, dy)
    counts = plan_arrays(p)["counts"].astype(np.int64)
    order = np.argsort(counts, kind="stable")
    live = order[counts[order] > 0]
    experts = [int(live[0]), int(live[len(live) // 2]), int(live[-8])]
    toks = np.unique(np.concatenate([[0, wl["T"] - 1], np.random.default_rng(2).choice(
        wl["T"], 22, replace=False)]))
    ref, _ = oracle_grads(wl, p, dy, 7.0, tokens=toks, experts=experts,
                          want=("dx", "dw"))
    close(g["dx"][toks], ref["dx"], "dx", dt)
    for key in ("dw_gate", "dw_up", "dw_down"):
        close(g[key][experts], ref[key], key, dt)


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
    ref, _ = oracle_grads(wl, p, dy, 7.0, want=("dx", "dtw"))
    close(g1["dx"], ref["dx"], "dx", dt)
    close(g1["d_topk_w"], ref["dtw"], "d_topk_w", dt)
