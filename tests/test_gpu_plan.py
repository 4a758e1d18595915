"""GPU plan (route + capacity + dispatch) against the oracle, bit-exactly:
ids, slots, keep/tok2pair, counts, offsets, the pair permutation and the
drop count, on every named workload, a capacity sweep and fuzzed shapes."""

import numpy as np
import pytest
import torch

import mixture_experts_routed_route_amd as moe
import oracle
import workloads as W
from helpers import check_plan, gpu_plan, plan_arrays, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,cf", [(1, None), (2, 1.5), (2, 3.0), (2, 6.0),
                                    (2, 0.0), (3, None), (4, None)])
def test_plan_named_workloads(cfg, cf):
    wl = W.config(cfg, capacity_factor=cf, with_weights=False)
    say(f"plan {wl['name']} cf={wl['capacity_factor']}")
    p = gpu_plan(wl)
    g, ref, st = check_plan(wl, p)
    if cfg == 2:
        expect_limit = {1.5: 48, 3.0: 96, 6.0: 192, 0.0: -1}[cf]
        assert st["limit"] == expect_limit
        if cf == 0.0:
            assert st["dropped"] == 0


@pytest.mark.parametrize("T", [33, 64, 128, 186])
def test_plan_short_prompts_shared(T):
    wl = W.config(5, T=T, with_weights=False)
    say(f"plan {wl['name']}")
    p = gpu_plan(wl)
    g, ref, st = check_plan(wl, p)
    assert g["counts"][128] == T


@pytest.mark.parametrize("ppe", range(1, 9))
def test_plan_exact_pairs_per_expert(ppe):
    wl = W.config(5, pairs_per_expert=ppe, with_weights=False)
    say(f"plan {wl['name']}")
    p = gpu_plan(wl)
    g, ref, st = check_plan(wl, p)
    assert np.all(g["counts"][:128] == ppe)


@pytest.mark.parametrize("T", [65, 128, 200, 256])
@pytest.mark.parametrize("E,k,cf", [(64, 8, 1.0), (256, 8, 0.0), (256, 2, 1.25),
                                    (16, 1, 2.0)])
def test_plan_prompts_of_65_to_256_tokens(T, E, k, cf):
    """Prompts just past the one-block plan's 64 tokens: the chunked plan's
    slot ranks cross chunk boundaries, and with a capacity limit they
    decide the drops (ranks counted on the histogram rows of earlier
    chunks)."""
    rng = np.random.default_rng(T * 7 + E + k)
    logits = (rng.standard_normal((T, E)) +
              1.5 * rng.standard_normal(E)).astype(np.float32)
    wl = dict(name=f"small{T}", T=T, E=E, k=k, n_shared=int(cf == 0.0),
              capacity_factor=cf, logits=torch.from_numpy(logits))
    say(f"plan T={T} E={E} k={k} cf={cf}")
    p = gpu_plan(wl)
    g, ref, st = check_plan(wl, p)
    if cf > 0:
        assert st["limit"] > 0


def _tie_heavy(T, E, rng):
    vals = np.array([-2.0, -0.0, 0.0, 0.5, 0.5, 1.0, 3.0], np.float32)
    return vals[rng.integers(0, len(vals), size=(T, E))]


@pytest.mark.parametrize("seed", range(12))
def test_plan_fuzz(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.choice([1, 2, 63, 64, 65, 127, 300, 1000, 4097]))
    E = int(rng.choice([1, 2, 3, 8, 63, 64, 65, 128, 200, 256, 513, 1024]))
    k = int(rng.integers(1, min(E, 16) + 1))
    if seed == 11:
        k = min(E, 70)          # more than one wave's worth of selections
    cf = float(rng.choice([0.0, 0.01, 0.5, 1.0, 1.25, 2.0, 8.0]))
    ns = int(rng.integers(0, 2))
    if seed % 3 == 0:
        logits = _tie_heavy(T, E, rng)
    else:
        logits = (rng.standard_normal((T, E)) +
                  2.0 * rng.standard_normal(E)).astype(np.float32)
    wl = dict(name=f"fuzz{seed}", T=T, E=E, k=k, n_shared=ns,
              capacity_factor=cf, logits=torch.from_numpy(logits))
    say(f"plan fuzz seed={seed} T={T} E={E} k={k} cf={cf} shared={ns}")
    p = gpu_plan(wl)
    check_plan(wl, p)


def test_plan_identical_rows_and_equal_logits():
    T, E, k = 130, 16, 4
    eq = torch.zeros(T, E)
    wl = dict(T=T, E=E, k=k, n_shared=0, capacity_factor=1.0, logits=eq)
    p = gpu_plan(wl)
    g, ref, st = check_plan(wl, p)
    assert np.all(g["topk_id"] == np.arange(k))
    assert np.all(g["topk_w"] == np.float32(0.25))
    lim = st["limit"]
    assert np.all(g["counts"][:k] == min(T, lim)) and np.all(g["counts"][k:] == 0)


def test_plan_nan_logits_rank_lowest():
    rng = np.random.default_rng(5)
    T, E, k = 70, 32, 3
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[rng.random((T, E)) < 0.1] = np.nan
    p = gpu_plan(dict(T=T, E=E, k=k, n_shared=0, capacity_factor=0.0,
                      logits=torch.from_numpy(lg)))
    st = moe.moe_plan_stats_get(p)
    assert st["nonfinite"] == int(np.isnan(lg).sum())
    ref = lg.copy()
    ref[np.isnan(ref)] = -np.inf   # NaN orders below every number
    ids, _ = oracle.route(ref, k)
    g = plan_arrays(p)
    assert np.array_equal(g["topk_id"], ids)


def test_plan_empty_prompt():
    wl = dict(T=0, E=8, k=2, n_shared=1, capacity_factor=1.0,
              logits=torch.zeros(0, 8))
    p = gpu_plan(wl)
    g = plan_arrays(p)
    assert np.all(g["offsets"] == 0)
    st = moe.moe_plan_stats_get(p)
    assert st["dropped"] == 0 and st["kept"] == 0 and st["drop_fraction"] == 0.0
