"""Seeded random layers against the oracle: prompt lengths on both sides of
the decode shape (16 tokens) and of the one-block plan (64 tokens), model
widths that leave ragged column blocks, expert counts from 1 to 64, top-k up
to 8, every dtype and 4-bit format, capacity caps, a shared expert, skewed
router biases, and forced switch points (S, fat_rows). Each case: the plan
bit for bit (ids, slots, counts, offsets, permutation) and the layer within
the dtype's bar on up to 48 sampled tokens. The cases are drawn once from a
fixed seed, so a failure names a reproducible case."""

import numpy as np
import pytest
import torch

import mixture_experts_routed_route_amd as moe
import workloads as W
from helpers import check_layer, check_plan, gpu_layer, oracle_layer, sample_tokens, say

pytestmark = pytest.mark.gpu


def _cases(n=48, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = ["bf16", "f16", "f32", "q4b32", "q4a32", "q4a64"][i % 6]
        T = int(rng.choice([1, 3, 9, 16, 17, 40, 64, 65, 130, 300, 513, 1031, 2049]))
        D = int(rng.choice([128, 256, 384, 512, 1024]))
        F = int(rng.choice([128, 256, 384, 640, 768]))
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        cf = float(rng.choice([0.0, 0.0, 1.0, 2.0]))
        ns = int(rng.integers(0, 2))
        spread = float(rng.choice([0.0, 1.0, 2.5]))
        S = rng.choice([None, None, 0.5, 8.0, 1e9]) if dt in ("bf16", "f16") else None
        fat = int(rng.choice([17, 64, 1000000])) if dt.startswith("q4") else None
        out.append(dict(i=i, dt=dt, T=T, D=D, F=F, E=E, k=k, cf=cf, ns=ns,
                        spread=spread, S=S, fat=fat, seed=int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("c", _cases(), ids=lambda c: f"case{c['i']}-{c['dt']}-T{c['T']}")
def test_random_layer_against_oracle(c):
    g = torch.Generator().manual_seed(c["seed"])
    bias = torch.randn(c["E"], generator=g) * c["spread"]
    x_dt = "f16" if c["dt"].startswith("q4") else c["dt"]
    w_dt = c["dt"] if c["dt"].startswith("q4") else None
    wl = W.make_layer(c["T"], c["D"], c["F"], c["E"], c["k"], x_dt, w_dtype=w_dt,
                      n_shared=c["ns"], logit_bias=bias, seed=c["seed"],
                      capacity_factor=c["cf"])
    say(f"fuzz {c}")
    opts = None
    if c["S"] is not None:
        opts = moe.make_options(splitk_max_pairs=float(c["S"]), exact_routes=True)
    elif c["fat"] is not None:
        opts = moe.make_options(fat_rows=c["fat"])
    p, y = gpu_layer(wl, options=opts)
    check_plan(wl, p)
    toks = sample_tokens(c["T"], 48, seed=c["i"]) if c["T"] > 48 else None
    check_layer(wl, y, toks, ref=oracle_layer(wl, toks))
