"""
Pins of the CPU oracle against things other than itself: a hand-worked
routing case (tests/golden), numpy brute force on tiny inputs, closed forms,
invariants of the layer, and library routines (numpy matmul/einsum/argsort,
numpy's float16 conversion, torch's bfloat16).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))


# ---------------------------------------------------------------- golden ---

def test_golden_route_plan_4x3():
    g = json.load(open(os.path.join(GOLDEN, "route_plan_4x3.json")))
    logits = np.array(g["logits"], np.float32)
    ids, w = oracle.route(logits, g["k"])
    assert ids.tolist() == g["ids"]
    want = []
    for item in g["weights_closed_form"]:
        want.append(0.5 if item[0] == "half" else sigmoid(item[1]))
    np.testing.assert_allclose(w.reshape(-1), want, rtol=0, atol=1e-15)
    for case in g["cases"]:
        pl = oracle.plan(ids, g["E"], case["capacity_factor"])
        assert pl["limit"] == case["limit"]
        assert pl["slot"].tolist() == case["slot"]
        assert pl["keep"].tolist() == case["keep"]
        assert pl["counts"].tolist() == case["counts"]
        assert pl["offsets"].tolist() == case["offsets"]
        assert pl["pair_token"].tolist() == case["pair_token"]
        assert pl["tok2pair"].tolist() == case["tok2pair"]
        assert pl["dropped"] == case["dropped"]
        assert pl["drop_fraction"] == case["drop_fraction"]
        # a token whose pairs all dropped gets exactly zero
        wl = W.make_layer(4, 32, 64, 3, 2, W.F32, logits=torch.tensor(logits),
                          seed=5)
        y = oracle.layer(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids,
                         w, pl["keep"], E=3, n_shared=0, x_dtype="f32",
                         w_dtype="f32", c=7.0)
        for t in range(4):
            assert (np.all(y[t] == 0.0)) == (t in case["zero_output_tokens"])


# --------------------------------------------------------------- routing ---

def _tie_heavy_logits(T, E, rng):
    # few distinct values, so ties at the k-th place are common; +-0 mixed
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 1.0, 2.0], np.float32)
    return vals[rng.integers(0, len(vals), size=(T, E))]


@pytest.mark.parametrize("seed", range(6))
def test_route_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 17))
    E = int(rng.integers(1, 9))
    k = int(rng.integers(1, E + 1))
    for logits in (rng.standard_normal((T, E)).astype(np.float32),
                   _tie_heavy_logits(T, E, rng)):
        ids, w = oracle.route(logits, k)
        bids, bw = brute.topk(logits, k)
        assert np.array_equal(ids, bids)
        np.testing.assert_allclose(w, bw, rtol=1e-12, atol=0)


def test_route_special_cases():
    T, E = 5, 16
    eq = np.zeros((T, E), np.float32)
    for k in (1, 2, 3, 8, 16):
        ids, w = oracle.route(eq, k)
        assert (ids == np.arange(k)).all()        # equal rows: 0..k-1
        assert (w == 1.0 / k).all()               # exactly 1/k
    lg = np.random.default_rng(1).standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route(lg, E)                  # k = E: all, descending
    for t in range(T):
        assert sorted(ids[t]) == list(range(E))
        assert np.all(np.diff(lg[t][ids[t]]) <= 0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    # two experts: w0 = sigmoid(l0 - l1)
    two = np.array([[1.5, -0.25], [0.0, 3.0]], np.float32)
    ids, w = oracle.route(two, 2)
    assert ids.tolist() == [[0, 1], [1, 0]]
    assert abs(w[0, 0] - sigmoid(1.75)) < 1e-15
    assert abs(w[1, 0] - sigmoid(3.0)) < 1e-15
    # +0 and -0 compare equal: the lower index wins
    z = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert oracle.route(z, 1)[0].tolist() == [[0]]
    with pytest.raises(ValueError):
        oracle.route(np.array([[np.nan, 0.0]], np.float32), 1)


# ---------------------------------------------------------- capacity/plan ---

@pytest.mark.parametrize("seed", range(8))
def test_plan_matches_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 17))
    E = int(rng.integers(1, 9))
    k = int(rng.integers(1, E + 1))
    logits = (rng.standard_normal((T, E)) + 2 * rng.standard_normal(E))
    ids, _ = oracle.route(logits.astype(np.float32), k)
    for cf in (0.0, 0.25, 0.5, 1.0, 1.5, 3.0, 1e9):
        pl = oracle.plan(ids, E, cf)
        slot, keep, counts, dropped = brute.capacity(ids, E, cf)
        assert np.array_equal(pl["slot"], slot)
        assert np.array_equal(pl["keep"].astype(bool), keep)
        assert np.array_equal(pl["counts"], counts)
        assert pl["dropped"] == dropped
        lim = brute.limit(T, E, k, cf)
        assert pl["limit"] == (-1 if lim is None else lim)
        # the pair permutation is a stable argsort of token-major expert ids,
        # restricted to the kept pairs
        flat = ids.reshape(-1)
        order = np.argsort(flat, kind="stable")
        kept_order = order[keep.reshape(-1)[order]]
        assert np.array_equal(pl["pair_src"], kept_order)
        assert np.array_equal(pl["pair_token"], kept_order // k)
        # inverse map
        t2p = pl["tok2pair"].reshape(-1)
        for pos, src in enumerate(pl["pair_src"]):
            assert t2p[src] == pos
        assert np.all(t2p[~keep.reshape(-1)] == -1)
        # the reported drop fraction is the count recomputed from the plan
        assert pl["drop_fraction"] == (T * k - pl["offsets"][E]) / (T * k)


def test_plan_invariants():
    rng = np.random.default_rng(7)
    T, E, k = 64, 8, 2
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route(logits, k)
    assert oracle.plan(ids, E, 0.0)["dropped"] == 0      # cf 0: no drops
    assert oracle.plan(ids, E, 1e6)["dropped"] == 0      # huge cf: none
    same = np.tile(logits[:1], (T, 1))                   # identical rows
    ids2, _ = oracle.route(same, k)
    for cf in (0.5, 1.0, 2.0):
        pl = oracle.plan(ids2, E, cf)
        lim = pl["limit"]
        for e in range(E):
            chosen = e in ids2[0]
            assert pl["counts"][e] == (min(T, lim) if chosen else 0)
    # limit reading: floor(cf*T*k/E), at least 1
    assert oracle.limit(2048, 128, 2, 1.5) == 48
    assert oracle.limit(2048, 128, 2, 3.0) == 96
    assert oracle.limit(2048, 128, 2, 6.0) == 192
    assert oracle.limit(10, 3, 1, 1.0) == 3
    assert oracle.limit(1, 1000, 1, 0.001) == 1
    assert oracle.limit(64, 8, 2, 0.0) == -1


def test_plan_shared_expert():
    rng = np.random.default_rng(3)
    T, E, k = 9, 6, 2
    ids, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    pl = oracle.plan(ids, E, 1.0, n_shared=1)
    assert pl["counts"][E] == T
    assert pl["offsets"][E + 1] - pl["offsets"][E] == T
    assert pl["pair_token"][pl["offsets"][E]:].tolist() == list(range(T))
    assert np.all(pl["pair_src"][pl["offsets"][E]:] == -1)
    # the shared expert is not counted in the drop fraction
    assert pl["drop_fraction"] == pl["dropped"] / (T * k)


# ------------------------------------------------------------ expert FFN ---

def _f64(t):
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("dt", [W.F32, W.BF16, W.F16])
def test_single_expert_top1_is_dense_swiglu(dt):
    wl = W.make_layer(12, 64, 96, 1, 1, dt, seed=11, w_std=0.2)
    ids, w = oracle.route(wl["logits"], 1)
    assert np.all(w == 1.0)
    pl = oracle.plan(ids, 1, 0.0)
    y = oracle.layer(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids, w,
                     pl["keep"], E=1, n_shared=0, x_dtype=dt, w_dtype=dt,
                     c=7.0)
    X, Wg, Wu, Wd = (_f64(wl[n]) for n in ("x", "w_gate", "w_up", "w_down"))
    G = np.minimum(X @ Wg[0].T, 7.0)
    U = np.clip(X @ Wu[0].T, -7.0, 7.0)
    ref = (G * (1.0 / (1.0 + np.exp(-G))) * U) @ Wd[0].T
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_all_experts_uncapped_is_dense_softmax_mixture():
    T, D, F, E = 10, 32, 48, 5
    wl = W.make_layer(T, D, F, E, E, W.F32, seed=12, w_std=0.3)
    ids, w = oracle.route(wl["logits"], E)
    pl = oracle.plan(ids, E, 0.0)
    y = oracle.layer(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids, w,
                     pl["keep"], E=E, n_shared=0, x_dtype="f32",
                     w_dtype="f32", c=0.0)
    X, Wg, Wu, Wd = (_f64(wl[n]) for n in ("x", "w_gate", "w_up", "w_down"))
    L = _f64(wl["logits"])
    P = np.exp(L - L.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    G = np.einsum("td,efd->tef", X, Wg)
    U = np.einsum("td,efd->tef", X, Wu)
    H = G / (1 + np.exp(-G)) * U
    Yall = np.einsum("tef,edf->ted", H, Wd)
    ref = np.einsum("te,ted->td", P, Yall)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_clamp_closed_form():
    # one-hot x; gate pre-activation 10, up pre-activation -10, clamp 7:
    # h = silu(min(10, 7)) * clip(-10, -7, 7) = 7*sigmoid(7) * -7
    D, F = 4, 2
    x = torch.tensor([1.0, 0.0, 0.0, 0.0])
    wg = torch.zeros(1, F, D)
    wu = torch.zeros(1, F, D)
    wd = torch.zeros(1, D, F)
    wg[0, 0, 0], wu[0, 0, 0] = 10.0, -10.0     # f = 0: both clamps bind
    wg[0, 1, 0], wu[0, 1, 0] = -10.0, 10.0     # f = 1: gate untouched below
    wd[0, 2, 0] = 1.0
    wd[0, 3, 1] = 1.0
    g, u, h, yp = oracle.expert(x, 0, wg, wu, wd, "f32", "f32", 7.0)
    assert g.tolist() == [10.0, -10.0] and u.tolist() == [-10.0, 10.0]
    assert abs(h[0] - (-49.0 * sigmoid(7.0))) < 1e-13
    assert abs(h[1] - (-10.0 * sigmoid(-10.0) * 7.0)) < 1e-13
    assert yp.tolist() == [0.0, 0.0, h[0], h[1]]
    # clamp 0 (off) and a huge clamp agree, and differ from c = 7
    _, _, h_off, _ = oracle.expert(x, 0, wg, wu, wd, "f32", "f32", 0.0)
    _, _, h_big, _ = oracle.expert(x, 0, wg, wu, wd, "f32", "f32", 1e30)
    assert h_off.tolist() == h_big.tolist()
    assert abs(h_off[0] - 10.0 * sigmoid(10.0) * -10.0) < 1e-12


def _layer(wl, cf, **kw):
    ids, w = oracle.route(wl["logits"], wl["k"])
    pl = oracle.plan(ids, wl["E"], cf, wl["n_shared"])
    y = oracle.layer(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids, w,
                     pl["keep"], E=wl["E"], n_shared=wl["n_shared"],
                     x_dtype=wl["x_dtype"], w_dtype=wl["w_dtype"], c=7.0, **kw)
    return ids, w, pl, y


@pytest.mark.parametrize("n_shared", [0, 1])
def test_layer_matches_dense_masked_bruteforce(n_shared):
    wl = W.make_layer(16, 32, 48, 6, 2, W.BF16, seed=13, w_std=0.3,
                      n_shared=n_shared,
                      logit_bias=torch.tensor([3.0, 2.0, 0, 0, -1, -2]))
    for cf in (0.0, 0.5, 1.0):
        ids, w, pl, y = _layer(wl, cf)
        if cf == 0.5:
            assert pl["dropped"] > 0
        X, Wg, Wu, Wd = (_f64(wl[n]) for n in ("x", "w_gate", "w_up",
                                               "w_down"))
        ref = brute.dense_layer(X, Wg, Wu, Wd, ids, w,
                                pl["keep"].astype(bool), 7.0, n_shared)
        np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_dropped_pairs_contribute_nothing():
    wl = W.make_layer(16, 32, 48, 4, 2, W.F32, seed=14, w_std=0.3,
                      logit_bias=torch.tensor([4.0, 0.0, 0.0, 0.0]))
    ids, w, pl, y = _layer(wl, 0.5)
    drop = pl["keep"] == 0
    assert drop.any()
    w2 = w.copy()
    w2[drop] = 123.0           # any weight on a dropped pair changes nothing
    y2 = oracle.layer(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids, w2,
                      pl["keep"], E=4, n_shared=0, x_dtype="f32",
                      w_dtype="f32", c=7.0)
    assert np.array_equal(y, y2)


def test_layer_linear_in_w_down_and_split_tokens():
    wl = W.make_layer(12, 32, 64, 4, 2, W.F32, seed=15, w_std=0.3)
    ids, w, pl, y = _layer(wl, 0.0)
    wl2 = dict(wl, w_down=wl["w_down"] * 4.0)   # exact in f32
    _, _, _, y2 = _layer(wl2, 0.0)
    np.testing.assert_allclose(y2, 4.0 * y, rtol=1e-12, atol=1e-14)
    # cf = 0: two calls over halves give the same rows as one call
    for half in (slice(0, 5), slice(5, 12)):
        part = dict(wl, logits=wl["logits"][half], x=wl["x"][half],
                    T=wl["x"][half].shape[0])
        _, _, _, yh = _layer(part, 0.0)
        np.testing.assert_array_equal(yh, y[half])
    # a token subset gives the same rows
    _, _, _, ys = _layer(wl, 0.0, tokens=[7, 2])
    np.testing.assert_array_equal(ys, y[[7, 2]])


# ----------------------------------------------------------- number formats ---

def test_f16_and_bf16_decode_match_library_casts():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.decode_f16_bits(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
    t = torch.randn(1, 8, 64).to(torch.bfloat16)
    d = oracle.decode(t, 0, "bf16")
    assert np.array_equal(d, t[0].to(torch.float64).numpy())


def test_q4_decode_ramp_and_nibble_order():
    # one row, 64 K values: block 0 ramps nibbles 0..15 twice, block 1 is
    # constant nibble 0x8 (-8); scales 0.5 and 2^-14 (smallest normal fp16)
    packed = np.zeros((1, 1, 32), np.uint8)
    for i in range(16):
        lo, hi = (2 * i) % 16, (2 * i + 1) % 16
        packed[0, 0, i] = lo | (hi << 4)
    packed[0, 0, 16:] = 0x88
    scales = np.array([[[0.5, 2.0 ** -14]]], np.float16)
    got = oracle.decode((torch.from_numpy(packed), torch.from_numpy(scales)),
                        0, "q4b32")[0]
    nib = [(kk % 16) for kk in range(32)]
    want0 = [(n - 16 if n >= 8 else n) * 0.5 for n in nib]
    assert got[:32].tolist() == want0
    assert got[32:].tolist() == [-8 * 2.0 ** -14] * 32
    # fp16(q*s) rounding: q*s exact, then round-to-nearest-even to fp16
    bits = oracle.dequant_q4_to_f16_bits(
        (torch.from_numpy(packed), torch.from_numpy(scales)), 0)
    assert np.array_equal(bits.view(np.float16).astype(np.float64)[0],
                          got)


def test_workload_sizes():
    # the five named workloads have the sizes the pages give (tiny ones only)
    wl = W.config(1)
    assert (wl["T"], wl["D"], wl["F"], wl["E"], wl["k"]) == (64, 128, 256, 8, 2)
    assert wl["x"].dtype == torch.float32
    p = W.config(5, pairs_per_expert=3)
    ids, _ = oracle.route(p["logits"], 8)
    pl = oracle.plan(ids, 128, 0.0, 1)
    assert np.all(pl["counts"][:128] == 3) and pl["counts"][128] == 48


def _numpy_q4_decode(packed, scales):
    """Independent vectorised unpack: low nibble first, two's complement."""
    p = packed.numpy()
    lo = (p & 15).astype(np.int64)
    hi = (p >> 4).astype(np.int64)
    q = np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)
    q = np.where(q >= 8, q - 16, q)
    s = np.repeat(scales.numpy().astype(np.float64), 32, axis=-1)
    return q * s


def test_q4_layer_matches_dense_bruteforce():
    wl = W.make_layer(8, 64, 96, 3, 2, W.F16, w_dtype=W.Q4B32, seed=16)
    for name in ("w_gate", "w_up", "w_down"):
        d = _numpy_q4_decode(*wl[name])
        for e in range(3):
            assert np.array_equal(oracle.decode(wl[name], e, "q4b32"), d[e])
    ids, w, pl, y = _layer(wl, 0.0)
    X = wl["x"].to(torch.float64).numpy()
    Wg, Wu, Wd = (_numpy_q4_decode(*wl[n]) for n in ("w_gate", "w_up",
                                                     "w_down"))
    ref = brute.dense_layer(X, Wg, Wu, Wd, ids, w, pl["keep"].astype(bool),
                            7.0)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dt,wdt", [(W.BF16, W.BF16), (W.F16, W.Q4B32),
                                    (W.F16, W.Q4A64)])
def test_pair_outputs_match_dense_experts(dt, wdt):
    # oracle.pairs on an arbitrary pair list (repeated tokens, every expert,
    # the shared slot, out of order) against numpy matmuls of independently
    # decoded weights, one expert at a time
    wl = W.make_layer(9, 128, 128, 4, 2, dt, w_dtype=wdt, seed=18, w_std=0.2,
                      n_shared=1)
    toks = np.array([8, 0, 3, 3, 5, 1, 8, 2])
    exps = np.array([4, 2, 0, 1, 3, 4, 0, 2])
    got = oracle.pairs(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], toks,
                       exps, x_dtype=dt, w_dtype=wdt, c=7.0)
    if wdt == W.Q4B32:
        Wg, Wu, Wd = (_numpy_q4_decode(*wl[n]) for n in ("w_gate", "w_up",
                                                         "w_down"))
    elif wdt == W.Q4A64:
        Wg, Wu, Wd = (_numpy_affine_decode(*wl[n], 64)
                      for n in ("w_gate", "w_up", "w_down"))
    else:
        Wg, Wu, Wd = (_f64(wl[n]) for n in ("w_gate", "w_up", "w_down"))
    X = _f64(wl["x"])
    for i, (t, e) in enumerate(zip(toks, exps)):
        ref = brute.expert_dense(X[t:t + 1], Wg[e], Wu[e], Wd[e], 7.0)[0]
        np.testing.assert_allclose(got[i], ref, rtol=1e-11, atol=1e-13)
    # the layer is the weighted sum of the kept pairs' outputs
    ids, w, pl, y = _layer(wl, 0.0)
    T, k = ids.shape
    tt = np.repeat(np.arange(T), k)
    yp = oracle.pairs(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], tt,
                      ids.reshape(-1), x_dtype=dt, w_dtype=wdt, c=7.0)
    sh = oracle.pairs(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"],
                      np.arange(T), np.full(T, 4), x_dtype=dt, w_dtype=wdt,
                      c=7.0)
    mix = (yp.reshape(T, k, -1) * w[:, :, None]).sum(1) + sh
    np.testing.assert_allclose(y, mix, rtol=1e-11, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.pairs(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], [9],
                     [0], x_dtype=dt, w_dtype=wdt, c=7.0)


@pytest.mark.parametrize("fmt,G", [("q4a32", 32), ("q4a64", 64)])
def test_q4_affine_decode_ramp_groups_and_rounding(fmt, G):
    # one row of 128 K values: nibble kk % 16 (low nibble = even index);
    # group j has scale 2^-j and bias -j - 0.25, so every group boundary
    # (each G values) changes both, and a swapped nibble or group index
    # changes the value
    K = 128
    packed = np.zeros((1, 1, K // 2), np.uint8)
    for i in range(K // 2):
        packed[0, 0, i] = ((2 * i) % 16) | (((2 * i + 1) % 16) << 4)
    ng = K // G
    params = np.zeros((1, 1, ng, 2), np.float16)
    for j in range(ng):
        params[0, 0, j] = (2.0 ** -j, -j - 0.25)
    w = (torch.from_numpy(packed), torch.from_numpy(params))
    got = oracle.decode(w, 0, fmt)[0]
    want = [(kk % 16) * 2.0 ** -(kk // G) - (kk // G) - 0.25 for kk in range(K)]
    assert got.tolist() == want
    # q*s + b rounded once to fp16: with s = 2^-14 * 3 and b = 1, q*s + b
    # needs more than fp16's 11 bits and rounds to nearest even
    params2 = np.zeros((1, 1, ng, 2), np.float16)
    params2[..., 0] = 3 * 2.0 ** -14
    params2[..., 1] = 1.0
    w2 = (torch.from_numpy(packed), torch.from_numpy(params2))
    exact = oracle.decode(w2, 0, fmt)[0]
    assert exact.tolist() == [(kk % 16) * 3 * 2.0 ** -14 + 1.0 for kk in range(K)]
    bits = oracle.dequant_q4_to_f16_bits(w2, 0, fmt)[0]
    ulp = 2.0 ** -10
    rounded = [math.floor(v / ulp + 0.5) * ulp if (v / ulp) % 1 != 0.5 else
               (math.floor(v / ulp) + (math.floor(v / ulp) % 2)) * ulp
               for v in exact.tolist()]
    assert bits.view(np.float16).astype(np.float64).tolist() == rounded


def _numpy_affine_decode(packed, params, G):
    p = packed.numpy()
    q = np.stack([p & 15, p >> 4], axis=-1).reshape(*p.shape[:-1], -1)
    pr = params.numpy().astype(np.float64)
    s = np.repeat(pr[..., 0], G, axis=-1)
    b = np.repeat(pr[..., 1], G, axis=-1)
    return q * s + b


@pytest.mark.parametrize("fmt,G", [(W.Q4A32, 32), (W.Q4A64, 64)])
def test_q4_affine_layer_matches_dense_bruteforce(fmt, G):
    wl = W.make_layer(8, 128, 192, 3, 2, W.F16, w_dtype=fmt, seed=17)
    for name in ("w_gate", "w_up", "w_down"):
        d = _numpy_affine_decode(*wl[name], G)
        for e in range(3):
            assert np.array_equal(oracle.decode(wl[name], e, fmt), d[e])
    ids, w, pl, y = _layer(wl, 0.0)
    X = wl["x"].to(torch.float64).numpy()
    Wg, Wu, Wd = (_numpy_affine_decode(*wl[n], G) for n in ("w_gate", "w_up",
                                                            "w_down"))
    ref = brute.dense_layer(X, Wg, Wu, Wd, ids, w, pl["keep"].astype(bool),
                            7.0)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


# ------------------------------------------------ router and statistics ---

def test_router_logits_hand_worked_product():
    # every value a small dyadic number, exact in bf16 and in the product
    x = torch.tensor([[1.0, 2.0], [3.0, -1.0]], dtype=torch.bfloat16)
    w = torch.tensor([[0.5, 0.25], [-1.0, 2.0], [4.0, 0.0]],
                     dtype=torch.bfloat16)
    out = oracle.router_logits(x, w, "bf16")
    assert out.tolist() == [[1.0, 3.0, 4.0], [1.25, -5.0, 12.0]]


def test_router_logits_one_hot_rows_read_columns():
    D, E = 40, 7
    w = (torch.randn(E, D, generator=torch.Generator().manual_seed(3))
         ).to(torch.float16)
    x = torch.eye(D, dtype=torch.float16)[[0, 5, 39]]
    out = oracle.router_logits(x, w, "f16")
    exact = oracle.decode_f16_bits(w.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(out, exact[:, [0, 5, 39]].T)


@pytest.mark.parametrize("E,k", [(16, 4), (256, 8), (5, 5)])
def test_router_stats_equal_logits(E, k):
    # p = 1/E everywhere: top-k mass k/E, the 0.9 mass needs ceil(0.9 E)
    # experts, lse = ln E, and every first choice is expert 0 (lower index),
    # so the balance term is E * 1 * (1/E) = 1
    T = 3
    st, want = oracle.router_stats(np.full((T, E), 0.75, np.float32), k, 0.5)
    lse = 0.75 + math.log(E)
    assert st["kept_mass"] == pytest.approx(k / E, rel=1e-14)
    assert want.tolist() == [math.ceil(0.9 * E)] * T
    assert st["z_loss"] == pytest.approx(lse * lse, rel=1e-14)
    assert st["balance"] == pytest.approx(1.0, rel=1e-14)
    assert st["aux"] == pytest.approx(1.0 + 0.5 * lse * lse, rel=1e-14)


@pytest.mark.parametrize("delta", [0.5, 2.0, 2.3, 3.0])
def test_router_stats_two_experts_closed_form(delta):
    # logits (delta, 0): p0 = sigmoid(delta); one expert holds 0.9 of the
    # mass iff p0 >= 0.9 (delta >= ln 9 = 2.197); lse = delta + ln(1 + e^-delta)
    lg = np.array([[delta, 0.0]] * 4, np.float32)
    d = float(np.float32(delta))
    p0 = sigmoid(d)
    st, want = oracle.router_stats(lg, 1, 1e-3)
    assert st["kept_mass"] == pytest.approx(p0, rel=1e-14)
    assert want.tolist() == [1 if p0 >= 0.9 else 2] * 4
    lse = d + math.log1p(math.exp(-d))
    assert st["z_loss"] == pytest.approx(lse * lse, rel=1e-14)
    assert st["balance"] == pytest.approx(2.0 * p0, rel=1e-14)


def test_router_stats_balanced_first_choice_gives_one():
    # first choices spread evenly: frac_e = 1/E, and the mean probabilities
    # sum to one whatever the logits, so the balance term is exactly 1
    E, T = 8, 64
    rng = np.random.default_rng(5)
    lg = rng.normal(size=(T, E)).astype(np.float32)
    lg[np.arange(T), np.arange(T) % E] += 20.0
    st, _ = oracle.router_stats(lg, 2, 0.0)
    assert st["balance"] == pytest.approx(1.0, rel=1e-13)
    assert st["aux"] == st["balance"]
    # all tokens on one expert: frac_0 = 1 and balance = E * mean p_0
    lg2 = rng.normal(size=(T, E)).astype(np.float32)
    lg2[:, 0] += 30.0
    st2, want2 = oracle.router_stats(lg2, 2, 0.0)
    p = np.exp(lg2.astype(np.float64) - lg2.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert st2["balance"] == pytest.approx(E * p[:, 0].mean(), rel=1e-13)
    assert want2.tolist() == [1] * T


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_router_stats_match_subset_bruteforce(seed):
    rng = np.random.default_rng(seed)
    T, E, k = 9, 7, 3
    lg = (rng.normal(size=(T, E)) * rng.uniform(0.3, 3.0)).astype(np.float32)
    lg[0, 1] = lg[0, 4]          # a tie on the first row
    st, want = oracle.router_stats(lg, k, 0.01)
    bst, bwant = brute.router_stats(lg, k, 0.01)
    assert want.tolist() == bwant.tolist()
    for key in oracle.ROUTER_STATS:
        assert st[key] == pytest.approx(bst[key], rel=1e-12), key


def test_router_stats_large_logits_stay_finite():
    # logits near 1000 overflow a naive exp; lse = 1000 + ln(1 + 2 + 4)
    lg = np.array([[1000.0 + math.log(4.0), 1000.0 + math.log(2.0), 1000.0]],
                  np.float32)
    st, want = oracle.router_stats(lg, 1, 1.0)
    l = lg.astype(np.float64)[0]
    lse = l[2] + math.log(math.exp(l[0] - l[2]) + math.exp(l[1] - l[2]) + 1.0)
    assert st["z_loss"] == pytest.approx(lse * lse, rel=1e-14)
    # the f32 logits hold 1000 + ln 4 to 6e-5: ratios from the stored values
    a, b = math.exp(l[0] - l[2]), math.exp(l[1] - l[2])
    assert st["kept_mass"] == pytest.approx(a / (a + b + 1.0), rel=1e-13)
    assert a / (a + b + 1.0) == pytest.approx(4.0 / 7.0, rel=1e-4)
    assert want.tolist() == [3]      # about 4/7 + 2/7 = 0.857 < 0.9


def test_router_stats_empty_and_nan():
    st, want = oracle.router_stats(np.zeros((0, 4), np.float32), 2)
    assert list(st.values()) == [0.0] * 5 and want.size == 0
    lg = np.zeros((2, 4), np.float32)
    lg[1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.router_stats(lg, 2)


# ------------------------------------------------------------- backward ---

def _autograd_dense(wl, ids, w, keep, dy, c):
    """The dense masked layer in torch float64 with autograd: every kept
    pair's FFN on its token, weighted, plus the shared expert; gradients of
    sum(dy * y) for x, the three weights and the routing weights."""
    T, D = wl["x"].shape
    E, ns = wl["E"], wl["n_shared"]
    x = wl["x"].to(torch.float64).clone().requires_grad_(True)
    Wg = torch.from_numpy(np.stack([oracle.decode(wl["w_gate"], e, wl["w_dtype"])
                                    for e in range(E + ns)])).requires_grad_(True)
    Wu = torch.from_numpy(np.stack([oracle.decode(wl["w_up"], e, wl["w_dtype"])
                                    for e in range(E + ns)])).requires_grad_(True)
    Wd = torch.from_numpy(np.stack([oracle.decode(wl["w_down"], e, wl["w_dtype"])
                                    for e in range(E + ns)])).requires_grad_(True)
    wt = torch.from_numpy(np.asarray(w, np.float64)).requires_grad_(True)

    def ffn(e, xr):
        g = Wg[e] @ xr
        u = Wu[e] @ xr
        if c > 0:
            g = torch.clamp(g, max=c)
            u = torch.clamp(u, -c, c)
        return Wd[e] @ (torch.nn.functional.silu(g) * u)

    rows = []
    for t in range(T):
        acc = torch.zeros(D, dtype=torch.float64)
        for j in range(ids.shape[1]):
            if keep[t, j]:
                acc = acc + wt[t, j] * ffn(int(ids[t, j]), x[t])
        if ns:
            acc = acc + ffn(E, x[t])
        rows.append(acc)
    y = torch.stack(rows)
    (y * torch.from_numpy(dy)).sum().backward()
    return dict(dx=x.grad.numpy(), dw_gate=Wg.grad.numpy(), dw_up=Wu.grad.numpy(),
                dw_down=Wd.grad.numpy(), dtw=wt.grad.numpy())


@pytest.mark.parametrize("n_shared,cf,c", [(0, 0.0, 7.0), (1, 1.0, 0.6),
                                           (0, 1.5, 0.0)])
def test_backward_matches_torch_autograd(n_shared, cf, c):
    # a tight clamp (0.6) binds on both g and u; cf 1 and 1.5 drop pairs
    wl = W.make_layer(12, 24, 20, 5, 2, W.BF16, seed=31, w_std=0.4,
                      n_shared=n_shared)
    ids, w = oracle.route(wl["logits"], 2)
    pl = oracle.plan(ids, 5, cf, n_shared)
    dy = np.random.default_rng(3).normal(size=(12, 24))
    got = oracle.backward(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids,
                          w, pl["keep"], dy, E=5, n_shared=n_shared,
                          x_dtype="bf16", w_dtype="bf16", c=c)
    ref = _autograd_dense(wl, ids, w, pl["keep"], dy, c)
    for key in ("dx", "dw_gate", "dw_up", "dw_down", "dtw"):
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-10, atol=1e-12,
                                   err_msg=key)
    if cf > 0:
        assert (pl["keep"] == 0).any()          # drops happened
        assert np.all(got["dtw"][pl["keep"] == 0] == 0)


def test_backward_subsets_match_full():
    wl = W.make_layer(10, 16, 12, 6, 3, W.F16, seed=32, w_std=0.3, n_shared=1)
    ids, w = oracle.route(wl["logits"], 3)
    pl = oracle.plan(ids, 6, 0.0, 1)
    dy = np.random.default_rng(4).normal(size=(10, 16))
    kw = dict(E=6, n_shared=1, x_dtype="f16", w_dtype="f16", c=7.0)
    full = oracle.backward(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids,
                           w, pl["keep"], dy, **kw)
    part = oracle.backward(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids,
                           w, pl["keep"], dy, tokens=[7, 2], experts=[6, 1],
                           want=("dx", "dw"), **kw)
    assert np.array_equal(part["dx"], full["dx"][[7, 2]])
    assert np.array_equal(part["dw_gate"], full["dw_gate"][[6, 1]])
    assert np.array_equal(part["dw_down"], full["dw_down"][[6, 1]])


def test_dlogits_central_differences():
    # L(logits) = sum(dy * layer(route(logits))) at cf 0; a small change of
    # the logits keeps the top-k choice, so dL/dl is the chain through the
    # renormalised weights
    wl = W.make_layer(4, 16, 12, 6, 3, W.BF16, seed=33, w_std=0.3)
    dy = np.random.default_rng(5).normal(size=(4, 16))
    kw = dict(E=6, n_shared=0, x_dtype="bf16", w_dtype="bf16", c=7.0)

    def loss(lg):
        ids, w = oracle.route(lg, 3)
        keep = np.ones((4, 3), np.uint8)
        y = oracle.layer(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids,
                         w, keep, **kw)
        return float((y * dy).sum()), ids

    lg0 = wl["logits"].numpy().astype(np.float32)
    ids, w = oracle.route(lg0, 3)
    g = oracle.backward(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids,
                        w, np.ones((4, 3), np.uint8), dy, want=("dtw",), **kw)
    dl = oracle.dlogits(ids, w, g["dtw"], 6)
    eps = 2.0 ** -10
    for t in range(4):
        for e in range(6):
            a, b = lg0.copy(), lg0.copy()
            a[t, e] += eps
            b[t, e] -= eps
            la, ia = loss(a)
            lb, ib = loss(b)
            assert np.array_equal(ia, ids) and np.array_equal(ib, ids)
            fd = (la - lb) / (2 * eps)
            assert fd == pytest.approx(dl[t, e], rel=2e-4, abs=1e-7), (t, e)
