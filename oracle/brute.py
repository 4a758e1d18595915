"""
TEST INFRASTRUCTURE ONLY: numpy brute force for tiny inputs.

Each function restates one step of the routed MoE layer in the most direct
form available, by a different route from ``moe_oracle.c``, so that the two
pin each other:

* ``topk`` sorts each row by (-logit, index) with Python's ``sorted``; the
  weights come from a full softmax over all E experts, then renormalised over
  the chosen k (the form the router uses on mini-AGI PR #3,
  minagi/pool.py, `requested(scores)`).
* ``capacity`` counts, for every pair, the earlier tokens that chose the same
  expert by an explicit O(T^2) scan, and keeps a pair while that count is
  under the limit (mini-AGI PR #3/#4, minagi/pool.py, the `keep` filter).
* ``dense_layer`` computes every expert on every token with numpy matmuls
  and mixes them with a dense [T, E] coefficient matrix that is zero for
  pairs not chosen or dropped, i.e. the single padded rectangle of mini-AGI
  PR #4 (minagi/pool.py, `experts()`), whose maths the grouped path must
  reproduce.
"""

from __future__ import annotations

import math

import numpy as np


def topk(logits: np.ndarray, k: int):
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    ids = np.zeros((T, k), np.int64)
    w = np.zeros((T, k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        ids[t] = order
        m = lg[t].max()
        p = np.exp(lg[t] - m)
        p = p / p.sum()
        sel = p[order]
        w[t] = sel / sel.sum()
    return ids, w


def limit(T: int, E: int, k: int, cf: float):
    """None when uncapped."""
    if cf == 0:
        return None
    return max(1, math.floor(cf * T * k / E))


def capacity(ids: np.ndarray, E: int, cf: float):
    """slot[T,k], keep[T,k], per-expert kept counts, dropped."""
    ids = np.asarray(ids)
    T, k = ids.shape
    lim = limit(T, E, k, cf)
    slot = np.zeros((T, k), np.int64)
    keep = np.zeros((T, k), bool)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            earlier = sum(1 for t2 in range(t) for j2 in range(k)
                          if ids[t2, j2] == e)
            slot[t, j] = earlier
            keep[t, j] = lim is None or earlier < lim
    counts = np.array([int(keep[ids == e].sum()) for e in range(E)])
    dropped = T * k - int(keep.sum())
    return slot, keep, counts, dropped


def expert_dense(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray,
                 Wd: np.ndarray, c: float) -> np.ndarray:
    """[n, D] -> [n, D]: silu(min(X Wg^T, c)) * clip(X Wu^T, -c, c) Wd^T."""
    G = X @ Wg.T
    U = X @ Wu.T
    if c > 0:
        G = np.minimum(G, c)
        U = np.clip(U, -c, c)
    H = G / (1.0 + np.exp(-G)) * U
    return H @ Wd.T


def dense_layer(X, Wg, Wu, Wd, ids, w, keep, c, n_shared=0):
    """Every expert on every token, mixed by a dense coefficient matrix."""
    X = np.asarray(X, np.float64)
    T = X.shape[0]
    E = Wg.shape[0] - n_shared
    coef = np.zeros((T, E))
    for t in range(T):
        for j in range(ids.shape[1]):
            if keep[t, j]:
                coef[t, ids[t, j]] += w[t, j]
    Y = np.zeros_like(X)
    for e in range(E):
        Y += coef[:, e:e + 1] * expert_dense(X, Wg[e], Wu[e], Wd[e], c)
    for s in range(n_shared):
        Y += expert_dense(X, Wg[E + s], Wu[E + s], Wd[E + s], c)
    return Y
