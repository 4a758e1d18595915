"""GPU layer output against the oracle on the same seeded inputs, within
max|y - ref| <= 2e-2 RMS(ref) (bf16/f16) or 1e-4 RMS(ref) (f32), on every
named workload, every route (split-K, full tile, dequant-once), forced route
switches, edge cases, and bit-exact dequantisation."""

import numpy as np
import pytest
import torch

import mixture_experts_routed_route_amd as moe
import oracle
import workloads as W
from helpers import (check_fat_copies, check_layer, check_pairs, check_plan,
                     gpu_layer, gpu_layer_views, gpu_plan, oracle_layer,
                     plan_arrays, sample_tokens, say, to_dev)

pytestmark = pytest.mark.gpu


def test_tiny_fp32_full():
    wl = W.config(1)
    say("layer tiny_fp32")
    p, y = gpu_layer(wl)
    check_plan(wl, p)
    check_layer(wl, y)


@pytest.mark.parametrize("cf", [1.5, 3.0, 6.0, 0.0])
def test_fresh_router_skew(cf):
    wl = W.config(2, capacity_factor=cf)
    say(f"layer fresh_router_skew cf={cf}")
    p, y = gpu_layer(wl)
    g, ref, st = check_plan(wl, p)
    toks = sample_tokens(wl["T"], 384, seed=int(cf * 10))
    check_layer(wl, y, toks)
    # tokens whose pairs all dropped come out exactly zero
    dead = np.where(ref["keep"].sum(1) == 0)[0]
    if len(dead):
        assert torch.all(y[torch.from_numpy(dead).cuda()] == 0)


def test_prefill_zipf():
    wl = W.config(3)
    say("layer prefill_zipf")
    p, y = gpu_layer(wl)
    check_layer(wl, y, sample_tokens(wl["T"], 160, seed=3))


@pytest.mark.parametrize("S", [0.0, 1e9])
def test_prefill_forced_routes(S):
    """All experts on the full tile (S=0) or all on split-K (S=1e9)."""
    wl = W.config(3)
    say(f"layer prefill_zipf S={S}")
    opts = moe.make_options(splitk_max_pairs=S, exact_routes=True)
    p, y = gpu_layer(wl, options=opts)
    check_layer(wl, y, sample_tokens(wl["T"], 96, seed=4))


@pytest.mark.parametrize("flag", ["plain", "split"])
@pytest.mark.parametrize("cfg", [3, 5])
def test_bf16_h_one_value_or_pair(cfg, flag):
    """The prefill and short-prompt layers with H forced to one bf16 value
    (the default for their uncapped plans) or to the hi + lo pair: both
    within the bar, every route (cfg 5 adds the shared expert)."""
    wl = W.config(cfg)
    f = moe.MOE_OPT_BF16_PLAIN_H if flag == "plain" else moe.MOE_OPT_BF16_SPLIT_H
    say(f"layer {wl['name']} bf16 H {flag}")
    p, y, views = gpu_layer_views(wl, options=moe.make_options(flags=f))
    assert ("h_lo" in views) == (flag == "split")
    counts = plan_arrays(p)["counts"]
    live = np.where(counts > 0)[0]
    check_pairs(wl, p, views, live[np.linspace(0, len(live) - 1, 6).astype(int)])
    check_layer(wl, y, sample_tokens(wl["T"], 96, seed=5))


@pytest.mark.parametrize("cf", [0.0, 1.25])
def test_bf16_h_default_follows_capacity(cf):
    """Without a flag, a bf16 layer carries H's low plane exactly when its
    plan is capped."""
    wl = W.make_layer(200, 256, 256, 16, 2, W.BF16, seed=29,
                      capacity_factor=cf, logit_bias=torch.linspace(2, -2, 16))
    p, y, views = gpu_layer_views(wl)
    assert ("h_lo" in views) == (cf > 0)
    check_layer(wl, y)


@pytest.mark.parametrize("T", [33, 64, 128, 186])
def test_short_prompt_shared(T):
    wl = W.config(5, T=T)
    say(f"layer {wl['name']}")
    p, y = gpu_layer(wl)
    check_layer(wl, y, sample_tokens(T, 64, seed=T))


@pytest.mark.parametrize("cfg,T", [(6, 1), (6, 2), (6, 4), (6, 8), (7, 1), (7, 8)])
def test_decode_shapes(cfg, T):
    # decode-shaped calls: k distinct experts per token, every touched
    # expert thin (one 16-row group), the shared expert too for cfg 6
    wl = W.config(cfg, T=T)
    say(f"layer {wl['name']}")
    p, y = gpu_layer(wl)
    check_plan(wl, p)
    check_layer(wl, y)


@pytest.mark.parametrize("T", [1, 5, 16])
@pytest.mark.parametrize("dt", [W.F32, W.F16])
def test_decode_groups_from_plan(dt, T):
    """Prompts of at most 16 tokens take the plan kernel's thin-group list
    instead of the classify kernel's (every expert holds at most T pairs);
    with a capacity cap some pairs drop, with S below T the classify kernel
    still decides (then experts may go to the full tile): all within the
    bar, plan bit-exact."""
    wl = W.make_layer(T, 256, 256, 16, 4, dt, seed=80 + T, capacity_factor=1.0,
                      n_shared=1, logit_bias=torch.linspace(1.5, -1.5, 16))
    say(f"layer decode groups {dt} T={T}")
    p, y = gpu_layer(wl)
    check_plan(wl, p)
    check_layer(wl, y)
    if dt != W.F32:
        p2, y2 = gpu_layer(wl, options=moe.make_options(splitk_max_pairs=0.5,
                                                        exact_routes=True))
        check_layer(wl, y2)


@pytest.mark.parametrize("exact", [False, True])
def test_underfilled_full_route(exact):
    # the shared expert (250 rows) and a few experts of 17..256 rows: their
    # full tiles (F / 128 = 2 column blocks each) cannot fill the GPU, so by
    # default they run as 64-row split-K groups; with exact routes, on the
    # full tile. Same plan, both within the bar, and equal to each other up
    # to summation order.
    bias = torch.zeros(16)
    bias[:3] = torch.tensor([4.0, 3.0, 2.5])
    wl = W.make_layer(250, 256, 256, 16, 2, W.BF16, seed=61, n_shared=1,
                      logit_bias=bias)
    say(f"layer underfilled full route exact={exact}")
    p, y = gpu_layer(wl, options=moe.make_options(exact_routes=exact))
    check_plan(wl, p)
    check_layer(wl, y)


@pytest.mark.parametrize("dt", [W.F16, W.BF16])
def test_full_tile_row_counts(dt):
    """Every expert on the full tile, with 426, 360, 204, 134, 94, 38, 19, 3
    and 2 rows: 256-row passes with ragged tails, the 128-row pass of tiles
    of at most 128 rows (the second tile of the 360-row expert, the small
    experts) and, for bf16, the split-H down passes; every token checked."""
    bias = torch.linspace(3.0, -3.0, 16)
    wl = W.make_layer(640, 256, 256, 16, 2, dt, seed=71, logit_bias=bias)
    say(f"layer full tile row counts {dt}")
    p, y = gpu_layer(wl, options=moe.make_options(splitk_max_pairs=0.0,
                                                  exact_routes=True))
    check_plan(wl, p)
    check_layer(wl, y)


@pytest.mark.parametrize("dt", [W.F16, W.BF16])
def test_full_tile_ragged_widths(dt):
    """d_model 384 and d_ff 640 on the full tile: the last 256-wide block
    of the down projection's outputs (and, for bf16, of the f32 rows it
    writes through LDS) is half outside d_model; every token checked."""
    bias = torch.linspace(2.0, -2.0, 8)
    wl = W.make_layer(400, 384, 640, 8, 2, dt, seed=73, logit_bias=bias)
    say(f"layer full tile D=384 F=640 {dt}")
    p, y = gpu_layer(wl, options=moe.make_options(splitk_max_pairs=0.0,
                                                  exact_routes=True))
    check_plan(wl, p)
    check_layer(wl, y)


@pytest.mark.parametrize("ppe", [1, 3, 4, 8])
@pytest.mark.parametrize("S", [0.0, 1e9])
def test_pairs_per_expert_both_tiles(ppe, S):
    wl = W.config(5, pairs_per_expert=ppe)
    say(f"layer {wl['name']} S={S}")
    p, y = gpu_layer(wl, options=moe.make_options(splitk_max_pairs=S,
                                                  exact_routes=True))
    check_layer(wl, y, sample_tokens(wl["T"], 24, seed=ppe))


def test_long_prompt_q4():
    """The 13,312-token 4-bit workload: the plan in full; the dequantised
    fp16 copies of three fat experts (first, middle, last slot) bit-exact as
    the forward's own dequant-once step wrote them; the per-pair output of
    every pair on a thin expert (split-K groups of <= 16 rows and the wide
    tile's 17..63) against the oracle; the layer output on sampled tokens."""
    wl = W.config(4)
    say("layer long_prompt_q4 (13312 tokens, 4-bit experts)")
    p, y, views = gpu_layer_views(wl)
    st = moe.moe_plan_stats_get(p)
    assert st["fat"] > 0 and st["touched"] > st["fat"]   # both routes used
    check_plan(wl, p)
    check_fat_copies(wl, p, views, 64, max_experts=3)
    counts = plan_arrays(p)["counts"]
    thin = np.where((counts > 0) & (counts < 64))[0]
    assert (counts[thin] <= 16).any() and (counts[thin] > 16).any()
    assert check_pairs(wl, p, views, thin) >= 1000
    check_layer(wl, y, sample_tokens(wl["T"], 40, seed=7))


@pytest.mark.parametrize("fat_rows", [0, 17, 64, 100000])
def test_q4_routes_small(fat_rows):
    """4-bit experts on the fat (dequant-once) and fused-dequant routes:
    every fat expert's fp16 copies bit-exact (gate/up K = 256, down K = 384:
    both decode tile depths), every pair's output, the layer."""
    wl = W.make_layer(520, 256, 384, 6, 2, W.F16, w_dtype=W.Q4B32, seed=21,
                      logit_bias=torch.tensor([3.0, 2.0, 1.0, 0.0, -2.0, -4.0]))
    say(f"layer q4 small fat_rows={fat_rows}")
    p, y, views = gpu_layer_views(wl, options=moe.make_options(fat_rows=fat_rows))
    counts = plan_arrays(p)["counts"]
    eff = 0 if fat_rows <= 0 else max(fat_rows, 17)
    if 0 < eff <= counts.max():
        assert len(check_fat_copies(wl, p, views, eff)) > 0
    check_pairs(wl, p, views, np.where(counts > 0)[0])
    check_layer(wl, y, sample_tokens(wl["T"], 64, seed=fat_rows % 97))


@pytest.mark.parametrize("dt", [W.BF16, W.F16, W.F32])
def test_edge_single_expert_top1(dt):
    wl = W.make_layer(77, 128, 256, 1, 1, dt, seed=22, w_std=0.05)
    say(f"layer E=1 k=1 {dt}")
    p, y = gpu_layer(wl)
    check_layer(wl, y)


def test_edge_all_experts_k_equals_E():
    wl = W.make_layer(65, 128, 128, 8, 8, W.BF16, seed=23, w_std=0.05,
                      n_shared=1)
    say("layer k=E with shared")
    p, y = gpu_layer(wl)
    check_layer(wl, y)


def test_edge_one_token_and_ragged():
    for T in (1, 2, 63, 65, 129):
        wl = W.make_layer(T, 256, 128, 16, 4, W.BF16, seed=24 + T,
                          capacity_factor=1.0)
        say(f"layer T={T}")
        p, y = gpu_layer(wl)
        check_plan(wl, p)
        check_layer(wl, y)


@pytest.mark.parametrize("S", [16.0, 64.0])
def test_stream_tile_row_blocks(S):
    # split-K experts of up to 64 rows: groups of 16 rows (S <= 16) or of
    # 64 rows in four token blocks (S > 16), bf16 hi + lo planes included
    wl = W.make_layer(600, 512, 256, 32, 2, W.BF16, seed=51, n_shared=1)
    say(f"layer stream tile S={S}")
    p, y = gpu_layer(wl, options=moe.make_options(splitk_max_pairs=S,
                                                  exact_routes=True))
    check_layer(wl, y, sample_tokens(wl["T"], 96, seed=3))


def test_q4_thin_groups_odd_width():
    # 4-bit thin experts with F = 384 (three 128-wide column blocks): groups
    # of <= 16 rows on the one-block split-K tile, 17..64 on the wide tile
    wl = W.make_layer(300, 512, 384, 16, 4, W.F16, w_dtype=W.Q4B32, seed=52)
    say("layer q4 F=384")
    p, y = gpu_layer(wl, options=moe.make_options(fat_rows=1000000))
    check_layer(wl, y, sample_tokens(wl["T"], 64, seed=4))


@pytest.mark.parametrize("dt,T", [(W.BF16, 1), (W.F16, 3), (W.Q4B32, 2)])
def test_thin_tiles_few_groups(dt, T):
    # a few thin groups: every (group, 128-row block) item of the 16-bit
    # stream tile spans several of its equal runs, so the fix-up adds partial
    # sums from three or more runs; 4-bit: the split-K tile on a few groups
    if dt == W.Q4B32:
        wl = W.make_layer(T, 1024, 512, 16, 4, W.F16, w_dtype=W.Q4B32,
                          seed=40 + T)
    else:
        wl = W.make_layer(T, 2048, 768, 16, 4, dt, seed=40 + T, n_shared=1)
    say(f"layer stream tile few groups {dt} T={T}")
    p, y = gpu_layer(wl)
    check_layer(wl, y)


@pytest.mark.parametrize("T,E,k", [(20, 16, 2), (40, 4, 2)])
def test_stream_tile_cut_items_many_runs(T, E, k):
    """Prompts just past the decode shape on few experts with d_model 2048:
    a stream launch holds a few hundred to a few thousand units (16 a
    128-row item), cut into runs of at least two, so an item spans 2 to 8
    runs and the run that arrives last adds that many partial sums inside
    the launch (the shared expert's 20 rows at T = 20: one group of 17..64
    rows, 12 items over 96 runs of two units); groups of <= 16 rows (one
    16-row block) and of 17..64 rows (four); the same bits run to run."""
    wl = W.make_layer(T, 2048, 768, E, k, W.BF16, seed=60 + T, n_shared=1)
    say(f"stream tile, items over many runs, T={T} E={E}")
    p, y = gpu_layer(wl)
    check_layer(wl, y)
    assert torch.equal(y, gpu_layer(wl)[1])


def test_edge_empty_prompt():
    wl = W.make_layer(0, 128, 128, 4, 2, W.BF16, seed=25)
    p, y = gpu_layer(wl)
    assert y.shape == (0, 128)


def test_edge_heavy_drop_zero_rows():
    bias = torch.tensor([8.0, 7.0] + [0.0] * 6)
    wl = W.make_layer(256, 128, 256, 8, 2, W.BF16, seed=26, logit_bias=bias,
                      capacity_factor=0.05)
    say("layer heavy drop")
    p, y = gpu_layer(wl)
    g, ref, st = check_plan(wl, p)
    assert st["drop_fraction"] > 0.5
    check_layer(wl, y)
    dead = np.where(ref["keep"].sum(1) == 0)[0]
    assert len(dead) > 0
    assert torch.all(y[torch.from_numpy(dead).cuda()] == 0)


def test_deterministic_and_routes_agree():
    wl = W.config(5, pairs_per_expert=6)
    a = gpu_layer(wl)[1]
    b = gpu_layer(wl)[1]
    assert torch.equal(a, b)                       # bitwise, run to run
    c = gpu_layer(wl, options=moe.make_options(splitk_max_pairs=0.0,
                                               exact_routes=True))[1]
    d = gpu_layer(wl, options=moe.make_options(splitk_max_pairs=1e9,
                                               exact_routes=True))[1]
    ref = oracle_layer(wl, sample_tokens(wl["T"], 32, seed=1))
    toks = sample_tokens(wl["T"], 32, seed=1)
    for y in (c, d):
        check_layer(wl, y, toks, ref=ref)
    # a route switch never changes the plan
    pa = gpu_plan(wl)
    pb = gpu_plan(wl)
    va, vb = moe.moe_plan_get_views(pa), moe.moe_plan_get_views(pb)
    for key in ("topk_id", "topk_w", "tok2pair", "pair_token"):
        assert torch.equal(va[key], vb[key])


@pytest.mark.parametrize("cfg", [3, 4])
def test_second_stream_matches_one_stream(cfg):
    """The thin groups' launches on the library's second stream (forked
    after the classification, joined before the combine) give the same
    bits as every launch on the caller's stream: the same kernels on
    disjoint rows, with the join ordering the combine after both."""
    wl = W.config(cfg)
    say(f"second stream vs one stream {wl['name']}")
    p = gpu_plan(wl)
    x = wl["x"].cuda()
    w = [to_dev(wl[n]) for n in ("w_gate", "w_up", "w_down")]
    two = moe.moe_forward(p, x, *w)
    one = moe.moe_forward(p, x, *w, options=moe.make_options(flags=moe.MOE_OPT_ONE_STREAM))
    two_again = moe.moe_forward(p, x, *w)
    torch.cuda.synchronize()
    assert torch.equal(two, one)
    assert torch.equal(two, two_again)


def test_phase_events_only_selected():
    """MOE_OPT_PHASE_ONLY bits limit the recorded phases to those selected
    (here the gate/up full tile); with none set every phase that ran is
    timed. The output is the same bits either way."""
    wl = W.config(3)
    say("phase events, selected and all")
    p = gpu_plan(wl)
    x = wl["x"].cuda()
    w = [to_dev(wl[n]) for n in ("w_gate", "w_up", "w_down")]
    moe.moe_phase_times(reset=True)
    one = moe.make_options(flags=moe.MOE_OPT_PHASE_EVENTS |
                           moe.MOE_OPT_PHASE_ONLY(moe.PHASES.index("gateup_full")))
    y1 = moe.moe_forward(p, x, *w, options=one)
    ms, calls = moe.moe_phase_times(reset=True)
    assert calls == 1
    assert ms["gateup_full"] > 0
    assert all(v == 0 for n, v in ms.items() if n != "gateup_full")
    y2 = moe.moe_forward(p, x, *w, options=moe.make_options(flags=moe.MOE_OPT_PHASE_EVENTS))
    ms2, calls2 = moe.moe_phase_times(reset=True)
    assert calls2 == 1
    for n in ("classify", "gateup_full", "down_full", "gateup_thin16", "combine"):
        assert ms2[n] > 0, n
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_swiglu_clamp_binds_and_matches():
    """Large weights so |g| > 7 often: the clamp decides the output."""
    wl = W.make_layer(96, 128, 256, 4, 2, W.F32, seed=27, w_std=0.9)
    p, y = gpu_layer(wl)
    check_layer(wl, y)
    # without the clamp the oracle result differs by far more than the bar
    ref_off = oracle_layer(dict(wl, swiglu_limit=0.0))
    yy = y.cpu().double().numpy()
    rms = np.sqrt(np.mean(ref_off ** 2))
    assert np.max(np.abs(yy - ref_off)) > 1e-2 * rms
    p2, y2 = gpu_layer(wl, options=moe.make_options(swiglu_limit=0.0))
    check_layer(dict(wl, swiglu_limit=0.0), y2)


def test_output_in_x_dtype_is_one_rounding_of_f32():
    """y in x's dtype equals the f32 output rounded once, bit for bit."""
    for dt in (W.BF16, W.F16):
        wl = W.make_layer(100, 128, 256, 8, 2, dt, seed=28, n_shared=1)
        p = gpu_plan(wl)
        y32 = gpu_layer(wl, plan=p)[1]
        x = wl["x"].cuda()
        yx = moe.moe_forward(p, x, wl["w_gate"].cuda(), wl["w_up"].cuda(),
                             wl["w_down"].cuda(), y_dtype=x.dtype)
        torch.cuda.synchronize()
        assert yx.dtype == x.dtype
        assert torch.equal(yx, y32.to(x.dtype))


@pytest.mark.parametrize("seed", [0, 1])
def test_dequant_once_bit_exact(seed):
    rng = np.random.default_rng(seed)
    E, N, K = 3, 48, 256
    packed = torch.from_numpy(rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8))
    sc = rng.uniform(0.005, 0.02, (E, N, K // 32))
    if seed == 1:
        # exercise rounding, fp16 subnormal results and large magnitudes
        sc = np.exp(rng.uniform(np.log(1e-6), np.log(4000.0), sc.shape))
    scales = torch.from_numpy(sc.astype(np.float16))
    out = moe.moe_dequant_q4(packed.cuda(), scales.cuda()).cpu()
    got = out.view(torch.int16).numpy().view(np.uint16)
    for e in range(E):
        want = oracle.dequant_q4_to_f16_bits((packed, scales), e)
        assert np.array_equal(got[e], want)
