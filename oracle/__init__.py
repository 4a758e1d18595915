"""
TEST INFRASTRUCTURE ONLY: the CPU oracle for the routed MoE FFN layer.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library and its Python binding
never do; the two share no code.

``moe_oracle.c`` (double precision, OpenMP) is the oracle proper; it is built
into ``liboracle.so`` next to it. ``brute.py`` holds independent numpy
restatements for tiny inputs that pin it. Parity status of every function is
listed below; all are pinned by tests in ``tests/test_oracle_*.py``:

  route / limit / plan / expert / pairs / layer / decode   pinned (brute force,
  closed forms, invariants, numpy library routines).
  backward / dlogits   pinned (torch float64 autograd of the dense masked
  layer; central differences of the oracle's own route + layer).
  router_logits / router_stats   pinned (a hand-worked product, one-hot rows,
  closed forms for equal logits and for two experts, a balanced first choice,
  subset enumeration on tiny inputs).
  The pages' own drop shares and speedups come from trained routers and
  other systems: parity unpinned (no input here reproduces them).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DT = {"f32": 0, "bf16": 1, "f16": 2, "q4b32": 3, "q4a32": 4, "q4a64": 5}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP, baseline x86-64)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                               "-std=c11", "-Wall", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or (os.path.getmtime(LIB)
                                       < os.path.getmtime(SRC)):
            build()
        L = ctypes.CDLL(LIB)
        i64, i32, dbl, vp = (ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                             ctypes.c_void_p)
        L.orc_route.argtypes = [i64, i32, i32, vp, vp, vp]
        L.orc_limit.argtypes = [i64, i32, i32, dbl]
        L.orc_limit.restype = i64
        L.orc_plan.argtypes = [i64, i32, i32, i32, dbl, vp, vp, vp, vp, vp,
                               vp, vp, vp, vp, vp]
        L.orc_expert.argtypes = [i64, i64, i64, vp, i32, vp, vp, vp, vp, vp,
                                 vp, i32, dbl, vp, vp, vp, vp]
        L.orc_layer.argtypes = [i64, i64, i64, i32, i32, i32, vp, i32, vp, vp,
                                vp, vp, vp, vp, i32, dbl, vp, vp, vp, i64, vp,
                                vp]
        L.orc_pairs.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, i32, vp,
                                vp, vp, vp, vp, vp, i32, dbl, vp]
        L.orc_decode.argtypes = [vp, vp, i32, i64, i64, i64, vp]
        L.orc_decode_f16.argtypes = [vp, i64, vp]
        L.orc_router_logits.argtypes = [i64, i64, i32, vp, i32, vp, vp]
        L.orc_router_stats.argtypes = [i64, i32, i32, vp, dbl, vp, vp]
        L.orc_backward.argtypes = [i64, i64, i64, i32, i32, i32, vp, i32, vp,
                                   vp, vp, vp, vp, vp, i32, dbl, vp, vp, vp,
                                   vp, i64, vp, vp, i32, vp, vp, vp, vp, vp]
        L.orc_dlogits.argtypes = [i64, i32, i32, vp, vp, vp, vp]
        L.orc_num_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _np(t):
    """A CPU tensor as a numpy array of its raw storage (16-bit as uint16)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t)
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _weight(w):
    """(data, scales) raw numpy arrays of one weight tensor or q4 pair."""
    if isinstance(w, (tuple, list)):
        return _np(w[0]), _np(w[1])
    return _np(w), None


def num_threads() -> int:
    return int(lib().orc_num_threads())


def route(logits, k: int):
    """ids [T, k] int32 (rank order) and weights [T, k] float64."""
    lg = np.ascontiguousarray(_np(logits), dtype=np.float32)
    T, E = lg.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    rc = lib().orc_route(T, E, k, _p(lg), _p(ids), _p(w))
    if rc != 0:
        raise ValueError(f"orc_route failed ({rc})")
    return ids, w


def router_logits(x, w_router, dtype: str) -> np.ndarray:
    """x [T, D] . w_router [E, D]^T in float64 over the stored values."""
    xa = _np(x)
    wa = _np(w_router)
    T, D = xa.shape
    E = wa.shape[0]
    out = np.zeros((T, E))
    rc = lib().orc_router_logits(T, D, E, _p(xa), DT[dtype], _p(wa), _p(out))
    if rc != 0:
        raise ValueError(f"orc_router_logits failed ({rc})")
    return out


ROUTER_STATS = ("kept_mass", "want_k", "z_loss", "balance", "aux")


def router_stats(logits, k: int, z_weight: float = 1e-3):
    """({kept_mass, want_k, z_loss, balance, aux} in float64, want per token)."""
    lg = np.ascontiguousarray(_np(logits), dtype=np.float32)
    T, E = lg.shape
    out = np.zeros(5)
    want = np.zeros(T, np.int32)
    rc = lib().orc_router_stats(T, E, k, _p(lg), float(z_weight), _p(out),
                                _p(want))
    if rc != 0:
        raise ValueError(f"orc_router_stats failed ({rc})")
    return dict(zip(ROUTER_STATS, out.tolist())), want


def limit(T: int, E: int, k: int, cf: float) -> int:
    """Capacity per expert; -1 means uncapped."""
    return int(lib().orc_limit(T, E, k, float(cf)))


def plan(ids: np.ndarray, E: int, cf: float, n_shared: int = 0) -> dict:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    P = T * k + n_shared * T
    out = dict(
        slot=np.zeros((T, k), np.int32), keep=np.zeros((T, k), np.uint8),
        counts=np.zeros(E + n_shared, np.int64),
        offsets=np.zeros(E + n_shared + 1, np.int64),
        pair_token=np.full(P, -1, np.int32), pair_src=np.full(P, -2, np.int32),
        tok2pair=np.zeros((T, k), np.int32))
    lim = np.zeros(1, np.int64)
    dropped = np.zeros(1, np.int64)
    rc = lib().orc_plan(T, E, k, n_shared, float(cf), _p(ids), _p(lim),
                        _p(out["slot"]), _p(out["keep"]), _p(out["counts"]),
                        _p(out["offsets"]), _p(out["pair_token"]),
                        _p(out["pair_src"]), _p(out["tok2pair"]), _p(dropped))
    if rc != 0:
        raise ValueError(f"orc_plan failed ({rc})")
    n = int(out["offsets"][-1])
    out["pair_token"] = out["pair_token"][:n]
    out["pair_src"] = out["pair_src"][:n]
    out["limit"] = int(lim[0])
    out["dropped"] = int(dropped[0])
    out["kept"] = T * k - int(dropped[0])
    out["drop_fraction"] = (int(dropped[0]) / (T * k)) if T * k else 0.0
    return out


def expert(x_row, e: int, w_gate, w_up, w_down, x_dtype: str, w_dtype: str,
           c: float):
    """g, u, h [F] and yp [D] of expert e on one token, in float64."""
    xr = _np(x_row).reshape(-1)
    D = xr.shape[0]
    wg, wgs = _weight(w_gate)
    wu, wus = _weight(w_up)
    wd, wds = _weight(w_down)
    F = wg.shape[1]
    g, u, h = (np.zeros(F) for _ in range(3))
    yp = np.zeros(D)
    rc = lib().orc_expert(D, F, e, _p(xr), DT[x_dtype], _p(wg), _p(wgs),
                          _p(wu), _p(wus), _p(wd), _p(wds), DT[w_dtype],
                          float(c), _p(g), _p(u), _p(h), _p(yp))
    if rc != 0:
        raise ValueError(f"orc_expert failed ({rc})")
    return g, u, h, yp


def pairs(x, w_gate, w_up, w_down, tokens, experts, *, x_dtype: str,
          w_dtype: str, c: float) -> np.ndarray:
    """Unweighted expert outputs yp [n, D] (float64) of the (tokens[i],
    experts[i]) pairs: FFN_e(x[t]) before the routing weight."""
    xa = _np(x)
    T, D = xa.shape
    wg, wgs = _weight(w_gate)
    wu, wus = _weight(w_up)
    wd, wds = _weight(w_down)
    F = wg.shape[1]
    n_exp = wg.shape[0]
    tl = np.ascontiguousarray(tokens, np.int64)
    el = np.ascontiguousarray(experts, np.int32)
    if tl.shape != el.shape or tl.ndim != 1:
        raise ValueError("tokens and experts must be 1-D and of one length")
    yp = np.zeros((tl.shape[0], D))
    rc = lib().orc_pairs(tl.shape[0], T, D, F, n_exp, _p(tl), _p(el), _p(xa),
                         DT[x_dtype], _p(wg), _p(wgs), _p(wu), _p(wus), _p(wd),
                         _p(wds), DT[w_dtype], float(c), _p(yp))
    if rc != 0:
        raise ValueError(f"orc_pairs failed ({rc})")
    return yp


def layer(x, w_gate, w_up, w_down, ids, w, keep, *, E: int, n_shared: int,
          x_dtype: str, w_dtype: str, c: float, tokens=None):
    """y [len(tokens) or T, D] float64 for the given routing and keep mask."""
    xa = _np(x)
    T, D = xa.shape
    wg, wgs = _weight(w_gate)
    wu, wus = _weight(w_up)
    wd, wds = _weight(w_down)
    F = wg.shape[1]
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    keep = np.ascontiguousarray(keep, np.uint8)
    k = ids.shape[1]
    tl = None if tokens is None else np.ascontiguousarray(tokens, np.int64)
    n = T if tl is None else tl.shape[0]
    y = np.zeros((n, D))
    rc = lib().orc_layer(T, D, F, E, k, n_shared, _p(xa), DT[x_dtype], _p(wg),
                         _p(wgs), _p(wu), _p(wus), _p(wd), _p(wds),
                         DT[w_dtype], float(c), _p(ids), _p(w), _p(keep), n,
                         _p(tl), _p(y))
    if rc != 0:
        raise ValueError(f"orc_layer failed ({rc})")
    return y


def backward(x, w_gate, w_up, w_down, ids, w, keep, dy, *, E: int,
             n_shared: int, x_dtype: str, w_dtype: str, c: float,
             tokens=None, experts=None, want=("dx", "dw", "dtw")) -> dict:
    """Gradients of L = sum(dy * y) in float64: dx [tokens or T, D], dw_gate /
    dw_up [experts or E + n_shared, F, D], dw_down [.., D, F], dtw [T, k]."""
    xa = _np(x)
    T, D = xa.shape
    wg, wgs = _weight(w_gate)
    wu, wus = _weight(w_up)
    wd, wds = _weight(w_down)
    F = wg.shape[1]
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    keep = np.ascontiguousarray(keep, np.uint8)
    dy = np.ascontiguousarray(_np(dy), np.float64)
    k = ids.shape[1]
    tl = None if tokens is None else np.ascontiguousarray(tokens, np.int64)
    el = None if experts is None else np.ascontiguousarray(experts, np.int32)
    nt = T if tl is None else tl.shape[0]
    ne = E + n_shared if el is None else el.shape[0]
    out = {}
    dx = np.zeros((nt, D)) if "dx" in want else None
    dwg = np.zeros((ne, F, D)) if "dw" in want else None
    dwu = np.zeros((ne, F, D)) if "dw" in want else None
    dwd = np.zeros((ne, D, F)) if "dw" in want else None
    dtw = np.zeros((T, k)) if "dtw" in want else None
    rc = lib().orc_backward(T, D, F, E, k, n_shared, _p(xa), DT[x_dtype],
                            _p(wg), _p(wgs), _p(wu), _p(wus), _p(wd), _p(wds),
                            DT[w_dtype], float(c), _p(ids), _p(w), _p(keep),
                            _p(dy), nt, _p(tl), _p(dx), ne, _p(el), _p(dwg),
                            _p(dwu), _p(dwd), _p(dtw))
    if rc != 0:
        raise ValueError(f"orc_backward failed ({rc})")
    out.update(dx=dx, dw_gate=dwg, dw_up=dwu, dw_down=dwd, dtw=dtw)
    return out


def dlogits(ids, w, dtw, E: int) -> np.ndarray:
    """Gradient of the logits [T, E] through the renormalised top-k weights."""
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    dtw = np.ascontiguousarray(dtw, np.float64)
    T, k = ids.shape
    out = np.zeros((T, E))
    lib().orc_dlogits(T, E, k, _p(ids), _p(w), _p(dtw), _p(out))
    return out


def decode(w, e: int, w_dtype: str) -> np.ndarray:
    """Expert e's [N, K] weight matrix decoded exactly to float64."""
    data, scales = _weight(w)
    N = data.shape[1]
    K = data.shape[2] * (2 if w_dtype.startswith("q4") else 1)
    out = np.zeros((N, K))
    rc = lib().orc_decode(_p(data), _p(scales), DT[w_dtype], e, N, K, _p(out))
    if rc != 0:
        raise ValueError(f"orc_decode failed ({rc})")
    return out


def decode_f16_bits(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, np.uint16)
    out = np.zeros(b.shape)
    lib().orc_decode_f16(_p(b), b.size, _p(out))
    return out


def dequant_q4_to_f16_bits(w, e: int, w_dtype: str = "q4b32") -> np.ndarray:
    """fp16 of expert e's 4-bit weights, rounded to nearest-even: uint16 bits
    [N, K].

    The value (q*s, or q*s + b for the affine groups) is exact in float64 (a
    4-bit integer times an fp16, plus an fp16), and numpy's float64 ->
    float16 cast rounds to nearest, ties to even.
    """
    exact = decode(w, e, w_dtype)
    return exact.astype(np.float16).view(np.uint16)


def run_workload(wl: dict, tokens=None) -> dict:
    """Route, plan and (for the given tokens) the layer output of a workload."""
    ids, w = route(wl["logits"], wl["k"])
    pl = plan(ids, wl["E"], wl["capacity_factor"], wl["n_shared"])
    y = layer(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids, w,
              pl["keep"], E=wl["E"], n_shared=wl["n_shared"],
              x_dtype=wl["x_dtype"], w_dtype=wl["w_dtype"],
              c=wl["swiglu_limit"], tokens=tokens)
    return dict(ids=ids, w=w, plan=pl, y=y)
