"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, and compare."""

from __future__ import annotations

import numpy as np
import torch

import mixture_experts_routed_route_amd as moe
import oracle

# Layer-output bars: max|y - ref| <= TOL * RMS(ref) (normwise, per token set).
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
# Gate weights: f32 on the GPU against f64 in the oracle.
W_RTOL = 1e-6


def say(*a):
    print(*a, flush=True)


def to_dev(w, dev="cuda"):
    if isinstance(w, (tuple, list)):
        return tuple(t.to(dev) for t in w)
    return w.to(dev)


def gpu_plan(wl, dev="cuda"):
    logits = wl["logits"].to(dev)
    p = moe.moe_plan_create(logits, wl["k"], wl["capacity_factor"],
                            wl["n_shared"])
    return p


def plan_arrays(p) -> dict:
    v = moe.moe_plan_get_views(p)
    torch.cuda.synchronize()
    return {k: t.cpu().numpy() for k, t in v.items()}


def check_plan(wl, p, ids_ref=None, w_ref=None):
    """Bit-exact routing/drop/permutation; weights within W_RTOL."""
    g = plan_arrays(p)
    if ids_ref is None:
        ids_ref, w_ref = oracle.route(wl["logits"], wl["k"])
    ref = oracle.plan(ids_ref, wl["E"], wl["capacity_factor"], wl["n_shared"])
    assert np.array_equal(g["topk_id"], ids_ref), "top-k ids differ"
    err = np.abs(g["topk_w"].astype(np.float64) - w_ref)
    assert np.all(err <= W_RTOL * np.abs(w_ref) + 1e-30), float(err.max())
    assert np.array_equal(g["slot"], ref["slot"]), "slots differ"
    assert np.array_equal(g["tok2pair"], ref["tok2pair"]), "tok2pair differs"
    assert np.array_equal(g["counts"], ref["counts"]), "counts differ"
    assert np.array_equal(g["offsets"], ref["offsets"]), "offsets differ"
    assert np.array_equal(g["pair_token"], ref["pair_token"]), "permutation"
    src = ref["pair_src"]
    pw_ref = np.where(src >= 0, w_ref.reshape(-1)[np.maximum(src, 0)], 1.0)
    assert np.all(np.abs(g["pair_w"] - pw_ref) <= W_RTOL * pw_ref + 1e-30)
    st = moe.moe_plan_stats_get(p)
    assert st["dropped"] == ref["dropped"]
    assert st["kept"] == ref["kept"]
    assert st["limit"] == ref["limit"]
    assert st["drop_fraction"] == ref["drop_fraction"]
    # the reported drop fraction is the count recomputed from the plan
    T, k = ids_ref.shape
    if T * k:
        assert st["drop_fraction"] == (T * k - g["offsets"][wl["E"]]) / (T * k)
    return g, ref, st


def gpu_layer(wl, options=None, dev="cuda", plan=None):
    p = plan if plan is not None else gpu_plan(wl, dev)
    x = wl["x"].to(dev)
    y = moe.moe_forward(p, x, to_dev(wl["w_gate"], dev), to_dev(wl["w_up"], dev),
                        to_dev(wl["w_down"], dev), options=options)
    torch.cuda.synchronize()
    return p, y


def oracle_layer(wl, tokens=None, ids=None, w=None, keep=None):
    if ids is None:
        ids, w = oracle.route(wl["logits"], wl["k"])
        pl = oracle.plan(ids, wl["E"], wl["capacity_factor"], wl["n_shared"])
        keep = pl["keep"]
    return oracle.layer(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids,
                        w, keep, E=wl["E"], n_shared=wl["n_shared"],
                        x_dtype=wl["x_dtype"], w_dtype=wl["w_dtype"],
                        c=wl["swiglu_limit"], tokens=tokens)


def sample_tokens(T, n, seed=0):
    if n >= T:
        return None
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(T, size=n, replace=False))
    # always include the first and last tokens (chunk edges, ragged tail)
    return np.unique(np.concatenate([[0, T - 1], idx]))


def check_layer(wl, y, tokens=None, ref=None):
    """max|y - ref| <= TOL * RMS(ref) over the checked tokens."""
    if ref is None:
        ref = oracle_layer(wl, tokens)
    yy = y.float().cpu().numpy().astype(np.float64)
    if tokens is not None:
        yy = yy[tokens]
    assert np.all(np.isfinite(yy)), "non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(yy - ref))) if ref.size else 0.0
    tol = TOL[wl["x_dtype"]]
    assert err <= tol * rms + 1e-30, f"max err {err:.3e} > {tol} x RMS {rms:.3e}"
    return err, rms


WDT = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "f16": moe.MOE_F16,
       "q4b32": moe.MOE_Q4B32, "q4a32": moe.MOE_Q4A32, "q4a64": moe.MOE_Q4A64}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def gpu_layer_views(wl, options=None, dev="cuda"):
    """The layer through the C ABI with an explicit forward workspace, and
    torch views of that workspace after the call (per-pair outputs, SwiGLU
    buffers, the dequantised fp16 copies of fat experts)."""
    p = gpu_plan(wl, dev)
    x = wl["x"].to(dev)
    wg, wu, wd = (to_dev(wl[n], dev) for n in ("w_gate", "w_up", "w_down"))
    o = options or moe.moe_options_default()
    D, F = wl["D"], wl["F"]
    xdt = TORCH_DT[wl["x_dtype"]]
    wdt = WDT[wl["w_dtype"]]
    nbytes = moe.moe_forward_workspace_bytes(p, D, F, WDT[wl["x_dtype"]], wdt, o)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    y = moe.moe_forward(p, x, wg, wu, wd, options=o, workspace=ws)
    torch.cuda.synchronize()
    views = moe.moe_forward_get_views(p, ws, D, F, xdt, wdt, o)
    return p, y, views


def check_fat_copies(wl, p, views, fat_rows, max_experts=None):
    """The fp16 copies the forward's dequantise-once step wrote, bit for bit
    against fp16_rne of the oracle's exact value (q * s, or q * s + b), for
    every fat expert (or the first, a middle and the last max_experts of
    them); the fat set is exactly the experts holding >= fat_rows pairs and
    the slots number them in expert order."""
    counts = plan_arrays(p)["counts"]
    fs = views["fat_slot"].cpu().numpy()
    fat = np.where(fs >= 0)[0]
    want_fat = np.where(counts >= fat_rows)[0] if fat_rows > 0 else fat[:0]
    assert np.array_equal(fat, want_fat), "fat experts differ"
    assert np.array_equal(fs[fat], np.arange(len(fat))), "fat slots"
    sel = fat
    if max_experts is not None and len(fat) > max_experts:
        idx = np.unique(np.linspace(0, len(fat) - 1, max_experts).astype(int))
        sel = fat[idx]
    D, F = wl["D"], wl["F"]
    dims = {"w_gate": (F, D), "w_up": (F, D), "w_down": (D, F)}
    for m, name in enumerate(("w_gate", "w_up", "w_down")):
        N, K = dims[name]
        for e in sel:
            got = views["fat_copy"][m][int(fs[e])].cpu().numpy().view(np.uint16)
            got = got.transpose(1, 0, 2).reshape(N, K)
            want = oracle.dequant_q4_to_f16_bits(wl[name], int(e), wl["w_dtype"])
            assert np.array_equal(got, want), f"{name} of expert {e}"
    return sel


def check_pairs(wl, p, views, experts, tol=None):
    """Every kept pair of the given experts: its unweighted expert output
    (the row the combine weighs) against the oracle's, max|err| <= TOL *
    RMS(ref) over the checked pairs."""
    a = plan_arrays(p)
    off, pt = a["offsets"], a["pair_token"]
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
    exps = np.concatenate([np.full(off[e + 1] - off[e], e) for e in experts])
    assert rows.size > 0
    ref = oracle.pairs(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"],
                       pt[rows], exps, x_dtype=wl["x_dtype"],
                       w_dtype=wl["w_dtype"], c=wl["swiglu_limit"])
    got = views["ypair"][torch.from_numpy(rows).cuda()].double().cpu().numpy()
    assert np.all(np.isfinite(got)), "non-finite pair output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)))
    t = TOL[wl["x_dtype"]] if tol is None else tol
    say(f"  {rows.size} pairs of {len(experts)} experts: max err / RMS = "
        f"{err / (rms + 1e-300):.2e}")
    assert err <= t * rms + 1e-30, f"pairs: max err {err:.3e} > {t} x RMS {rms:.3e}"
    return rows.size
