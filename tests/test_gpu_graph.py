"""Plan + forward captured once into a HIP graph (torch.cuda.CUDAGraph) and
replayed on new inputs: every replay must give what the eager calls give on
the same inputs, bit for bit (the same kernels, deterministic). Between the
replays the test runs its own eager work and synchronises, and each replay
gets new logits (so new routes, pair lists and route classes) and new x,
copied into the captured input buffers. Covers decode calls of 1 and 8
tokens on the 16-bit and the 4-bit layers, a short prompt with a shared
expert, and the prefill layer (full tile with its work-queue counters,
which the path clears with a kernel, not a memset)."""

import pytest
import torch

import mixture_experts_routed_route_amd as moe
import workloads as W
from helpers import say, to_dev

pytestmark = pytest.mark.gpu

CASES = [(6, 1), (6, 8), (7, 1), (7, 8), (5, 128), (3, None)]


def _eager(wl, logits, x, w):
    p = moe.moe_plan_create(logits, wl["k"], wl["capacity_factor"], wl["n_shared"])
    return moe.moe_forward(p, x, *w)


@pytest.mark.parametrize("cfg,T", CASES)
def test_graph_replays_match_eager(cfg, T):
    wl = W.config(cfg, T=T)
    say(f"graph capture {wl['name']} T={wl['T']}")
    Tn, D, F, E, k, ns = (wl[n] for n in ("T", "D", "F", "E", "k", "n_shared"))
    cf = wl["capacity_factor"]
    w = [to_dev(wl[n]) for n in ("w_gate", "w_up", "w_down")]
    wdt = moe.MOE_BF16 if wl["w_dtype"] == "bf16" else (
        moe.MOE_F16 if wl["w_dtype"] == "f16" else moe.MOE_Q4B32)
    xdt = {"bf16": moe.MOE_BF16, "f16": moe.MOE_F16}[wl["x_dtype"]]
    logits_s = wl["logits"].cuda().clone()
    x_s = wl["x"].cuda().clone()
    plan_ws = torch.empty(moe.moe_plan_workspace_bytes(Tn, E, k, cf, ns),
                          dtype=torch.uint8, device="cuda")
    p0 = moe.moe_plan_create(logits_s, k, cf, ns, workspace=plan_ws)
    fwd_ws = torch.empty(moe.moe_forward_workspace_bytes(p0, D, F, xdt, wdt),
                         dtype=torch.uint8, device="cuda")
    y_g = torch.empty(Tn, D, dtype=torch.float32, device="cuda")

    def step():
        p = moe.moe_plan_create(logits_s, k, cf, ns, workspace=plan_ws)
        moe.moe_forward(p, x_s, *w, out=y_g, workspace=fwd_ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i in range(4):
        # new inputs, copied into the captured buffers (the first replay
        # keeps the captured ones): the experts' logits rotated (other
        # routes and loads) and x's features rotated
        if i > 0:
            logits_s.copy_(torch.roll(wl["logits"], 7 * i, dims=1).cuda())
            x_s.copy_(torch.roll(wl["x"], 13 * i, dims=1).cuda())
        ref = _eager(wl, logits_s.clone(), x_s.clone(), w)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, ref), f"replay {i}: max diff {(y_g - ref).abs().max().item()}"
        # eager work between replays, on the default stream
        ref2 = _eager(wl, logits_s, x_s, w)
        torch.cuda.synchronize()
        assert torch.equal(ref2, ref)
    del g
