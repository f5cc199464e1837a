"""Oracle: decode attention and the split-K combine (test infrastructure only).

[Cross] §1 and §4.1 have dense and sparse modes read their caches through one
split-K decoding kernel; §4.4 shows why that fixed dense path matters.  What
the kernel computes is plain softmax attention of the step's query heads over
a set of cached rows -- the full cache (dense mode) or the gathered buffer
(KV mode) -- so the oracle is that definition written out in float64:

    z_j   = q_h . k_{h//G, j} * scale
    out_h = sum_j softmax(z)_j v_{h//G, j}
    lse_h = log sum_j exp(z_j)

Splitting the rows into chunks and merging the chunk results by
log-sum-exp only reaches the same numbers faster; `combine` is the merge rule
written out on its own so that the GPU's merge can be checked in isolation.
An empty chunk is (m = -inf, l = 0, acc = 0) and contributes nothing.

Ragged lengths (one row count per KV head, for per-head budgets) are the
same definition applied head by head.

Pins (tests/test_oracle_attention.py): brute-force loops on tiny inputs,
weights sum to one, constant V gives that constant, a single row gives that
row, q = 0 gives the mean of V, combining any partition of the rows
reproduces the unsplit result, and ragged lengths equal the per-head
brute-force loops.
"""

from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_rows: int,
           scale: float) -> tuple[np.ndarray, np.ndarray]:
    """q [h_q, d_h]; k, v [h_kv, >= n_rows, d_h] -> out [h_q, d_h], lse [h_q]."""
    h_q, d_h = q.shape
    h_kv = k.shape[0]
    if h_q % h_kv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = h_q // h_kv
    out = np.empty((h_q, d_h), dtype=np.float64)
    lse = np.empty(h_q, dtype=np.float64)
    for h in range(h_q):
        kk = k[h // g, :n_rows].astype(np.float64)
        vv = v[h // g, :n_rows].astype(np.float64)
        z = kk @ q[h].astype(np.float64) * scale
        m = z.max()
        e = np.exp(z - m)
        l = e.sum()
        out[h] = (e @ vv) / l
        lse[h] = m + np.log(l)
    return out, lse


def attend_ragged(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads,
                  scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Ragged per-head lengths: the query heads of KV head kv attend over its
    rows 0..n_heads[kv]-1 (a gathered buffer with one budget per head)."""
    h_q, d_h = q.shape
    h_kv = k.shape[0]
    g = h_q // h_kv
    out = np.empty((h_q, d_h), dtype=np.float64)
    lse = np.empty(h_q, dtype=np.float64)
    for kv in range(h_kv):
        o, l = attend(q[kv * g:(kv + 1) * g], k[kv:kv + 1], v[kv:kv + 1], int(n_heads[kv]), scale)
        out[kv * g:(kv + 1) * g] = o
        lse[kv * g:(kv + 1) * g] = l
    return out, lse


def partials(q, k, v, bounds, scale):
    """Chunk partials (m, l, acc) for chunks [bounds[s], bounds[s+1])."""
    h_q, d_h = q.shape
    g = h_q // k.shape[0]
    n_chunks = len(bounds) - 1
    m = np.full((h_q, n_chunks), -np.inf)
    l = np.zeros((h_q, n_chunks))
    acc = np.zeros((h_q, n_chunks, d_h))
    for h in range(h_q):
        for s in range(n_chunks):
            a, b = bounds[s], bounds[s + 1]
            if b <= a:
                continue
            kk = k[h // g, a:b].astype(np.float64)
            vv = v[h // g, a:b].astype(np.float64)
            z = kk @ q[h].astype(np.float64) * scale
            m[h, s] = z.max()
            e = np.exp(z - m[h, s])
            l[h, s] = e.sum()
            acc[h, s] = e @ vv
    return m, l, acc


def combine(m: np.ndarray, l: np.ndarray, acc: np.ndarray):
    """Merge chunk partials: out = sum_s e^{m_s-M} acc_s / sum_s e^{m_s-M} l_s."""
    big = m.max(axis=1, keepdims=True)
    wgt = np.where(np.isfinite(m), np.exp(m - big), 0.0)
    den = (wgt * l).sum(axis=1)
    out = (wgt[:, :, None] * acc).sum(axis=1) / den[:, None]
    lse = big[:, 0] + np.log(den)
    return out, lse


def attend_loops(q, k, v, n_rows, scale):
    """Pure-Python twin of `attend` for tiny inputs."""
    import math
    h_q, d_h = q.shape
    g = h_q // k.shape[0]
    out = np.zeros((h_q, d_h))
    lse = np.zeros(h_q)
    for h in range(h_q):
        kv = h // g
        z = [sum(float(q[h, c]) * float(k[kv, j, c]) for c in range(d_h)) * scale
             for j in range(n_rows)]
        mx = max(z)
        e = [math.exp(x - mx) for x in z]
        tot = sum(e)
        for c in range(d_h):
            out[h, c] = sum(e[j] * float(v[kv, j, c]) for j in range(n_rows)) / tot
        lse[h] = mx + math.log(tot)
    return out, lse
