"""
Seeded synthetic inputs for the routed mixture-of-experts FFN layer.

This module is shared by the CPU oracle (under ``oracle/``), the HIP path's
tests and the benchmark. It only draws numbers: it holds none of the layer's
arithmetic (no top-k, no capacity rule, no expert FFN, no combine).

Every workload is a plain dict of CPU torch tensors plus its sizes:

* ``logits``  f32 [T, E] router logits (bf16-valued where the layer runs in
  bf16, so that ties at the k-th place really occur),
* ``x``       [T, D] activations in the layer's dtype (f32, bf16 or f16),
* ``w_gate``, ``w_up`` [E + n_shared, F, D] and ``w_down`` [E + n_shared, D, F]
  expert weights, K-contiguous, in the layer's dtype; for 4-bit weights each is
  a pair ``(packed u8 [.., N, K/2], scales f16 [.., N, K/32])`` — two's
  complement nibbles, the low nibble holding the even K index, one fp16 scale
  per 32 consecutive K values.

The five named workloads follow the sizes of the routed-MoE pages:
a tiny fp32 layer; a fresh router with per-expert bias so a few "sink" experts
take most rows (mini-AGI PR #3, configs/strix_halo_large.yaml
``capacity_factor`` comment, and PR #4 ``minagi/pool.py`` "GROUPED BY LOAD"
comment); a Zipf-skewed prefill layer; a 13K-token prompt over 4-bit experts
(Strata PR #4366, "Problem and result"); and short prompts with a shared
expert and an exact number of pairs per expert (TensorFold PR #1607, "What
this changes" and "Why 3.5, and why a fraction").
"""

from __future__ import annotations

import torch

F32, BF16, F16, Q4B32 = "f32", "bf16", "f16", "q4b32"
Q4A32, Q4A64 = "q4a32", "q4a64"
Q4_FORMATS = (Q4B32, Q4A32, Q4A64)

_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}

CONFIG_NAMES = {
    1: "tiny_fp32",
    2: "fresh_router_skew",
    3: "prefill_zipf",
    4: "long_prompt_q4",
    5: "short_prompt_shared",
    6: "decode_shared",
    7: "decode_q4",
}


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def _normal(shape, std, g):
    return torch.randn(*shape, generator=g) * std


def _random_bytes(n: int, g: torch.Generator) -> torch.Tensor:
    """n uniform random bytes (so each nibble is uniform on 0..15)."""
    words = (n + 7) // 8
    r = torch.randint(-(2 ** 63), 2 ** 63 - 1, (words,), dtype=torch.int64,
                      generator=g)
    return r.view(torch.uint8)[:n].clone() if words * 8 != n else r.view(torch.uint8)


def zipf_bias(E: int, s: float, g: torch.Generator) -> torch.Tensor:
    """Per-expert logit bias b_e = -s * ln(1 + pi(e)), pi a seeded permutation.

    Under softmax this makes expert popularity fall off as rank^-s.
    """
    perm = torch.randperm(E, generator=g).to(torch.float64)
    return (-s * torch.log1p(perm)).to(torch.float32)


def round_robin_logits(T: int, E: int, k: int, g: torch.Generator) -> torch.Tensor:
    """Token t favours experts (k*t + j) mod E for j < k by a wide margin.

    With T a multiple of E/k every expert then holds exactly T*k/E pairs.
    Inside the favoured set the bonus descends with j, so the top-k order is
    fixed; the noise is far smaller than the margins.
    """
    base = torch.randn(T, E, generator=g) * 0.1
    t = torch.arange(T).unsqueeze(1)
    j = torch.arange(k).unsqueeze(0)
    cols = (k * t + j) % E
    bonus = 20.0 + (k - j).to(torch.float32)
    base.scatter_(1, cols, base.gather(1, cols) + bonus.expand(T, k))
    return base


def as_dtype(a: torch.Tensor, dtype: str) -> torch.Tensor:
    return a.to(_TORCH_DTYPE[dtype]).contiguous()


def dense_weights(E_total: int, D: int, F: int, std: float, dtype: str,
                  g: torch.Generator):
    """Gate/up [E, F, D] and down [E, D, F], N(0, std), in the given dtype."""
    wg = as_dtype(_normal((E_total, F, D), std, g), dtype)
    wu = as_dtype(_normal((E_total, F, D), std, g), dtype)
    wd = as_dtype(_normal((E_total, D, F), std, g), dtype)
    return wg, wu, wd


def q4_weights(E_total: int, N: int, K: int, g: torch.Generator,
               scale_lo: float = 0.005, scale_hi: float = 0.02):
    """4-bit block weights [E, N, K]: uniform nibbles, fp16 scales ~U(lo, hi)."""
    assert K % 32 == 0
    packed = _random_bytes(E_total * N * K // 2, g).view(E_total, N, K // 2)
    scales = torch.empty(E_total, N, K // 32).uniform_(scale_lo, scale_hi,
                                                      generator=g)
    return packed, scales.to(torch.float16).contiguous()


def q4_affine_weights(E_total: int, N: int, K: int, group: int,
                      g: torch.Generator, scale_lo: float = 0.005,
                      scale_hi: float = 0.02):
    """Affine 4-bit weights [E, N, K]: uniform unsigned nibbles and per group
    of ``group`` K values an fp16 scale ~U(lo, hi) and bias (-7.5 + U(-1, 1))
    * scale, interleaved as [E, N, K / group, 2] (scale, bias)."""
    assert K % group == 0
    packed = _random_bytes(E_total * N * K // 2, g).view(E_total, N, K // 2)
    ng = K // group
    scales = torch.empty(E_total, N, ng).uniform_(scale_lo, scale_hi, generator=g)
    shift = torch.empty(E_total, N, ng).uniform_(-1.0, 1.0, generator=g)
    params = torch.stack([scales, (shift - 7.5) * scales], dim=-1)
    return packed, params.to(torch.float16).contiguous()


def make_layer(T: int, D: int, F: int, E: int, k: int, dtype: str, *,
               w_dtype: str | None = None, n_shared: int = 0,
               logits: torch.Tensor | None = None, logit_bias=None,
               bf16_logits: bool = False, x_std: float = 1.0,
               w_std: float = 0.02, seed: int = 0, capacity_factor=0.0,
               swiglu_limit: float = 7.0, name: str = "custom",
               with_weights: bool = True) -> dict:
    """A seeded layer instance. The draw order is fixed: logits, x, weights.

    ``with_weights=False`` draws the logits alone (identical to the full
    draw's logits), for plan-only uses of the large workloads.
    """
    g = _gen(seed)
    w_dtype = w_dtype or dtype
    if logits is None:
        logits = torch.randn(T, E, generator=g)
        if logit_bias is not None:
            logits = logits + logit_bias
    if bf16_logits:
        logits = logits.to(torch.bfloat16).to(torch.float32)
    logits = logits.to(torch.float32).contiguous()
    base = dict(name=name, T=T, D=D, F=F, E=E, k=k, n_shared=n_shared,
                x_dtype=dtype, w_dtype=w_dtype or dtype, logits=logits,
                capacity_factor=float(capacity_factor),
                swiglu_limit=float(swiglu_limit), seed=seed)
    if not with_weights:
        return base
    x = as_dtype(_normal((T, D), x_std, g), dtype)
    Et = E + n_shared
    if w_dtype == Q4B32:
        wg = q4_weights(Et, F, D, g)
        wu = q4_weights(Et, F, D, g)
        wd = q4_weights(Et, D, F, g)
    elif w_dtype in (Q4A32, Q4A64):
        grp = 32 if w_dtype == Q4A32 else 64
        wg = q4_affine_weights(Et, F, D, grp, g)
        wu = q4_affine_weights(Et, F, D, grp, g)
        wd = q4_affine_weights(Et, D, F, grp, g)
    else:
        wg, wu, wd = dense_weights(Et, D, F, w_std, w_dtype, g)
    return dict(base, x=x, w_gate=wg, w_up=wu, w_down=wd)


def config(n: int, *, seed: int = 0, capacity_factor=None, T=None,
           pairs_per_expert=None, with_weights: bool = True,
           w_dtype: str | None = None) -> dict:
    """The five named workloads (sizes from the routed-MoE pages).

    1 tiny fp32: T=64, D=128, F=256, E=8, top-2, cf 0.
    2 fresh-router skew: T=2048, D=512, F=1024, E=128, top-2, bf16, logits
      N(0,1) + per-expert bias N(0, 2^2); cf in {1.5, 3, 6, 0} (default 1.5).
    3 prefill: T=4096, D=2048, F=768, E=128, top-8, bf16, Zipf(1.1) bias.
    4 long prompt, 4-bit experts: T=13312, D=4096, F=2048, E=256, top-8,
      x f16, q4 weights with fp16 block scales ~U(0.005, 0.02), Zipf(1.1).
    5 short prompt + shared expert: D=2048, F=768, E=128, top-8 + 1 shared,
      bf16; T in {33, 64, 128, 186} with N(0,1) logits, or, given
      ``pairs_per_expert`` p, T = 16p with round-robin logits so every
      routed expert holds exactly p pairs.
    6 decode on the layer of 5: T in 1..8 (default 1), N(0,1) logits.
    7 decode on the layer of 4: T in 1..8 (default 1), Zipf(1.1) bias.

    ``w_dtype`` (4 and 7 only) swaps the 4-bit format: "q4a64" / "q4a32"
    give affine 4-bit weights (groups of 64 / 32, fp16 scale and bias) of
    the same shapes; the name gets the format as a suffix.
    """
    if w_dtype not in (None, Q4B32) and n not in (4, 7):
        raise ValueError("w_dtype applies to the 4-bit workloads 4 and 7")
    wq = w_dtype or Q4B32
    suffix = "" if wq == Q4B32 else "_" + wq
    if n == 1:
        return make_layer(64, 128, 256, 8, 2, F32, seed=seed,
                          capacity_factor=capacity_factor or 0.0,
                          name=CONFIG_NAMES[1], with_weights=with_weights)
    if n == 2:
        g = _gen(seed + 1000)
        bias = torch.randn(128, generator=g) * 2.0
        cf = 1.5 if capacity_factor is None else capacity_factor
        return make_layer(2048, 512, 1024, 128, 2, BF16, logit_bias=bias,
                          bf16_logits=True, seed=seed, capacity_factor=cf,
                          name=CONFIG_NAMES[2], with_weights=with_weights)
    if n == 3:
        g = _gen(seed + 1000)
        bias = zipf_bias(128, 1.1, g)
        return make_layer(4096, 2048, 768, 128, 8, BF16, logit_bias=bias,
                          bf16_logits=True, seed=seed,
                          capacity_factor=capacity_factor or 0.0,
                          name=CONFIG_NAMES[3], with_weights=with_weights)
    if n == 4:
        g = _gen(seed + 1000)
        bias = zipf_bias(256, 1.1, g)
        return make_layer(13312, 4096, 2048, 256, 8, F16, w_dtype=wq,
                          logit_bias=bias, seed=seed,
                          capacity_factor=capacity_factor or 0.0,
                          name=CONFIG_NAMES[4] + suffix,
                          with_weights=with_weights)
    if n == 5:
        if pairs_per_expert is not None:
            p = int(pairs_per_expert)
            T5 = 16 * p
            logits = round_robin_logits(T5, 128, 8, _gen(seed + 2000 + p))
            logits = logits.to(torch.bfloat16).to(torch.float32)
            return make_layer(T5, 2048, 768, 128, 8, BF16, n_shared=1,
                              logits=logits, seed=seed,
                              name=f"{CONFIG_NAMES[5]}_p{p}",
                              with_weights=with_weights)
        T5 = 128 if T is None else int(T)
        return make_layer(T5, 2048, 768, 128, 8, BF16, n_shared=1,
                          bf16_logits=True, seed=seed,
                          name=f"{CONFIG_NAMES[5]}_T{T5}",
                          with_weights=with_weights)
    if n == 6:
        # decode-shaped calls on the short-prompt layer: T in 1..8 tokens
        T6 = 1 if T is None else int(T)
        return make_layer(T6, 2048, 768, 128, 8, BF16, n_shared=1,
                          bf16_logits=True, seed=seed,
                          name=f"{CONFIG_NAMES[6]}_T{T6}",
                          with_weights=with_weights)
    if n == 7:
        # decode-shaped calls on the 4-bit layer: T in 1..8 tokens
        T7 = 1 if T is None else int(T)
        g = _gen(seed + 1000)
        bias = zipf_bias(256, 1.1, g)
        return make_layer(T7, 4096, 2048, 256, 8, F16, w_dtype=wq,
                          logit_bias=bias, seed=seed,
                          name=f"{CONFIG_NAMES[7]}_T{T7}{suffix}",
                          with_weights=with_weights)
    raise ValueError(f"no workload {n}")


def make_router(T: int, D: int, E: int, k: int, dtype: str, *, seed: int = 0,
                capacity_factor: float = 0.0, n_shared: int = 0,
                spread: float = 0.0) -> dict:
    """Inputs of the router map: x [T, D] ~ N(0, 1) and its weight [E, D]
    with rows ~ N(0, s_e^2 / D), so each logit is about N(0, s_e^2). s_e = 1,
    or with ``spread`` > 0 a seeded log-uniform factor exp(spread * U(-1, 1))
    per expert, so a few wide experts win most first choices."""
    g = _gen(seed)
    x = as_dtype(_normal((T, D), 1.0, g), dtype)
    scale = torch.ones(E, 1)
    if spread > 0:
        scale = torch.exp((torch.rand(E, 1, generator=g) * 2 - 1) * spread)
    w = as_dtype(_normal((E, D), 1.0 / D ** 0.5, g) * scale, dtype)
    return dict(T=T, D=D, E=E, k=k, dtype=dtype, x=x, w_router=w,
                capacity_factor=capacity_factor, n_shared=n_shared)


def flops_per_pair(D: int, F: int) -> int:
    """Multiply-adds counted as 2 flops: gate, up and down products."""
    return 6 * D * F


def weight_bytes_per_expert(D: int, F: int, w_dtype: str) -> float:
    per = {F32: 4.0, BF16: 2.0, F16: 2.0, Q4B32: 0.5 + 2.0 / 32.0,
           Q4A32: 0.5 + 4.0 / 32.0, Q4A64: 0.5 + 4.0 / 64.0}[w_dtype]
    return 3.0 * D * F * per


def dtype_bytes(dtype: str) -> int:
    return {F32: 4, BF16: 2, F16: 2}[dtype]

