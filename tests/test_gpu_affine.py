"""Affine 4-bit weights (unsigned nibbles, an fp16 scale and bias per group of
32 or 64 K values) on the GPU against the oracle: the dequant-once values
bit-exact (fp16_rne(q * s + b)), and the layer on the fat (dequant-once),
split-K and wide fused-dequant routes within the fp16 bar."""

import numpy as np
import pytest
import torch

import mixture_experts_routed_route_amd as moe
import oracle
import workloads as W
from helpers import (check_fat_copies, check_layer, check_pairs, check_plan,
                     gpu_layer, gpu_layer_views, plan_arrays, sample_tokens,
                     say)

pytestmark = pytest.mark.gpu

FORMATS = [W.Q4A32, W.Q4A64]


@pytest.mark.parametrize("fmt", [W.Q4B32, W.Q4A32, W.Q4A64])
@pytest.mark.parametrize("K", [256, 384])
def test_dequant_weights_bit_exact(fmt, K):
    g = torch.Generator().manual_seed(K + len(fmt))
    if fmt == W.Q4B32:
        w = W.q4_weights(3, 40, K, g)
    else:
        w = W.q4_affine_weights(3, 40, K, 32 if fmt == W.Q4A32 else 64, g)
    say(f"dequant {fmt} K={K}")
    out = moe.moe_dequant_weights(w[0].cuda(), w[1].cuda())
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    for e in range(3):
        assert np.array_equal(got[e], oracle.dequant_q4_to_f16_bits(w, e, fmt)), e


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("fat_rows", [0, 17, 64, 100000])
def test_affine_routes_small(fmt, fat_rows):
    """fat (dequant-once + full tile), split-K and wide tiles; F = 384 makes
    the down stage's K = 384 (128-deep chunks and a 128-value tail step, and
    the dequant-once step's 4-block tiles): the fat copies bit-exact, every
    pair's output, the layer."""
    wl = W.make_layer(520, 256, 384, 6, 2, W.F16, w_dtype=fmt, seed=121,
                      logit_bias=torch.tensor([3.0, 2.0, 1.0, 0.0, -2.0, -4.0]))
    say(f"layer {fmt} small fat_rows={fat_rows}")
    p, y, views = gpu_layer_views(wl, options=moe.make_options(fat_rows=fat_rows))
    counts = plan_arrays(p)["counts"]
    eff = 0 if fat_rows <= 0 else max(fat_rows, 17)
    if 0 < eff <= counts.max():
        assert len(check_fat_copies(wl, p, views, eff)) > 0
    check_pairs(wl, p, views, np.where(counts > 0)[0])
    check_layer(wl, y, sample_tokens(wl["T"], 64, seed=fat_rows % 97))


@pytest.mark.parametrize("fmt", FORMATS)
def test_affine_thin_groups_odd_width(fmt):
    wl = W.make_layer(300, 512, 384, 16, 4, W.F16, w_dtype=fmt, seed=152)
    say(f"layer {fmt} F=384 thin")
    p, y = gpu_layer(wl, options=moe.make_options(fat_rows=1000000))
    check_layer(wl, y, sample_tokens(wl["T"], 64, seed=4))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("T", [1, 2, 8])
def test_affine_decode_shapes(fmt, T):
    wl = W.config(7, T=T, w_dtype=fmt)
    say(f"layer {wl['name']}")
    p, y = gpu_layer(wl)
    check_plan(wl, p)
    check_layer(wl, y)


def test_long_prompt_affine_g64():
    """The 13,312-token layer with affine 4-bit groups of 64: the fp16 copies
    of three fat experts bit-exact, every thin pair's output, sampled
    tokens."""
    wl = W.config(4, w_dtype=W.Q4A64)
    say("layer long_prompt_q4_q4a64 (13312 tokens, affine 4-bit, groups of 64)")
    p, y, views = gpu_layer_views(wl)
    st = moe.moe_plan_stats_get(p)
    assert st["fat"] > 0 and st["touched"] > st["fat"]
    check_fat_copies(wl, p, views, 64, max_experts=3)
    counts = plan_arrays(p)["counts"]
    check_pairs(wl, p, views, np.where((counts > 0) & (counts < 64))[0])
    check_layer(wl, y, sample_tokens(wl["T"], 40, seed=8))
