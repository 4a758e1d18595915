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
* ``router_stats`` recomputes the routing statistics of mini-AGI PR #3
  (minagi/pool.py, `requested(scores)`) with Python floats: the experts a
  token "wants" by enumerating every subset of experts (the smallest size
  of a subset holding 0.9 of the mass), the first choices by a counting
  dictionary, the log-sum-exp with ``math.fsum``.
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


def router_stats(logits: np.ndarray, k: int, z_weight: float):
    """(dict of the five statistics, want per token); tiny E only (2^E)."""
    from itertools import combinations
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    firsts = {}
    kept = want = zsum = 0.0
    mean_p = [0.0] * E
    wants = []
    for t in range(T):
        row = [float(v) for v in lg[t]]
        m = max(row)
        ex = [math.exp(v - m) for v in row]
        tot = math.fsum(ex)
        p = [v / tot for v in ex]
        lse = m + math.log(tot)
        zsum += lse * lse
        order = sorted(range(E), key=lambda e: (-row[e], e))
        kept += math.fsum(p[e] for e in order[:k])
        firsts[order[0]] = firsts.get(order[0], 0) + 1
        for e in range(E):
            mean_p[e] += p[e] / T
        need = E
        for size in range(1, E + 1):
            if any(math.fsum(p[e] for e in sub) >= 0.9
                   for sub in combinations(range(E), size)):
                need = size
                break
        wants.append(need)
        want += need
    balance = E * math.fsum((firsts.get(e, 0) / T) * mean_p[e]
                            for e in range(E))
    z = zsum / T
    return (dict(kept_mass=kept / T, want_k=want / T, z_loss=z,
                 balance=balance, aux=balance + z_weight * z),
            np.array(wants, np.int32))
