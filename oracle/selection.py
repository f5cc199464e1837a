"""Oracle: one-time attention-scored KV selection (test infrastructure only).

[Cross] §4.1 describes the KV branch as SnapKV-style: right after a dense
prefill, the cache is scored once with the attention of the last prompt
queries (the observation window), a few sink tokens plus the best-scoring
entries of each KV head are kept up to a keep ratio, and the kept entries are
gathered into one contiguous buffer that later steps read and extend.

Readings where the page is silent or garbled:

* Window size w is a parameter (the page's text says 64; [CateKV] B.1 gives 32
  for SnapKV; the workloads here use 32).
* Score of entry j for KV head kv: the sum, over the w window queries and over
  the G query heads that share kv, of the causal softmax weight that the query
  puts on j.  Query i of the window sits at position p = n - w + i and sees
  keys 0..p; logits are q . k / sqrt(d_h).  No pooling or smoothing.
* Query head h reads KV head h // G (grouped-query attention).
* Forced entries: sinks [0, n_sink) and the window [n - w, n) are always kept;
  the remaining k_keep - n_sink - w slots go to the largest scores among
  [n_sink, n - w), ties to the lower position; the kept list is ascending.
* k_keep >= n keeps everything (a keep ratio of 1 disables the branch,
  [Cross] §5.3).
* The sink-plus-recent window ([Cross] §4.1, §4.4) keeps the first n_sink
  rows and the most recent rows up to the same count, read in place.

The top-k decision is taken on float32 scores (the precision of the HIP
kernels; the page fixes none), so that both sides decide identically when
they are handed the same float32 array.

* Ragged budgets (CateKV-style hybrid retention): each KV head has its own
  k_keep and follows the same rule; which heads are adaptive is an input (the
  page classifies heads offline from reference data).

Pins (tests/test_oracle_selection.py): softmax rows sum to one so the scores of
a KV head sum to G*w; brute-force Python loops on tiny inputs; identity at
k_keep >= n; all-equal scores pick the lowest positions; planted high-logit
keys are recovered; ragged budgets equal to one k reproduce the uniform
selection head by head; the CateKV budgets' kept fraction in closed form.  Output parity on random data beyond these invariants is
unpinned: the selection is a heuristic defined by the steps above.
"""

from __future__ import annotations

import numpy as np


def _group(n_q_heads: int, n_kv_heads: int) -> int:
    if n_q_heads % n_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    return n_q_heads // n_kv_heads


def window_logits(q_win: np.ndarray, k: np.ndarray, n: int, scale: float,
                  h: int) -> np.ndarray:
    """z[i, j] = q_{h,i} . k_{h//G, j} * scale, with -inf where j > n - w + i."""
    w = q_win.shape[1]
    g = _group(q_win.shape[0], k.shape[0])
    z = (q_win[h].astype(np.float64) @ k[h // g, :n].astype(np.float64).T) * scale
    pos = n - w + np.arange(w)[:, None]
    z[np.arange(n)[None, :] > pos] = -np.inf
    return z


def window_lse(q_win: np.ndarray, k: np.ndarray, n: int, scale: float) -> np.ndarray:
    """log-sum-exp of each window query over its causal prefix: [h_q, w]."""
    h_q, w = q_win.shape[:2]
    out = np.empty((h_q, w), dtype=np.float64)
    for h in range(h_q):
        z = window_logits(q_win, k, n, scale, h)
        m = z.max(axis=1, keepdims=True)
        out[h] = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    return out


def window_scores(q_win: np.ndarray, k: np.ndarray, n: int, scale: float) -> np.ndarray:
    """S[kv, j]: summed causal softmax weights of the window queries: [h_kv, n]."""
    h_q = q_win.shape[0]
    h_kv = k.shape[0]
    g = _group(h_q, h_kv)
    lse = window_lse(q_win, k, n, scale)
    s = np.zeros((h_kv, n), dtype=np.float64)
    for h in range(h_q):
        z = window_logits(q_win, k, n, scale, h)
        s[h // g] += np.exp(z - lse[h][:, None]).sum(axis=0)
    return s


def select_indices(scores_f32: np.ndarray, n: int, w: int, n_sink: int,
                   k_keep: int) -> np.ndarray:
    """Kept positions per KV head, ascending: int32 [h_kv, min(k_keep, n)].

    `scores_f32` must be float32 [h_kv, >= n]; the ranking compares those float32
    values exactly, larger first, equal values ordered by position.
    """
    scores_f32 = np.asarray(scores_f32)
    if scores_f32.dtype != np.float32:
        raise TypeError("selection decides on float32 scores")
    h_kv = scores_f32.shape[0]
    if k_keep >= n:
        return np.tile(np.arange(n, dtype=np.int32), (h_kv, 1))
    if w > n or n_sink < 0 or k_keep < n_sink + w:
        raise ValueError("need w <= n and k_keep >= n_sink + w")
    m = k_keep - n_sink - w
    cand = np.arange(n_sink, n - w)
    out = np.empty((h_kv, k_keep), dtype=np.int32)
    for kv in range(h_kv):
        s = scores_f32[kv, n_sink:n - w].astype(np.float64)
        order = np.lexsort((cand, -s))  # primary: larger score; secondary: lower j
        chosen = cand[order[:m]]
        keep = np.concatenate([np.arange(n_sink), chosen, np.arange(n - w, n)])
        out[kv] = np.sort(keep)
    return out


def select_indices_ragged(scores_f32: np.ndarray, n: int, w: int, n_sink: int,
                          k_heads) -> list:
    """Per-KV-head budgets: KV head kv keeps k_heads[kv] entries by the rule of
    select_indices (CateKV's hybrid retention, "CateKV: On Sequential
    Consistency for Long-Context LLM Inference Acceleration", §3 "CateKV Cache
    Policy": a few critical entries for consistent heads, most for adaptive
    heads).  Returns one ascending int32 array per head, min(k, n) long."""
    scores_f32 = np.asarray(scores_f32)
    return [select_indices(scores_f32[kv:kv + 1], n, w, n_sink, int(k))[0]
            for kv, k in enumerate(k_heads)]


def catekv_budgets(n: int, adaptive, budget: int, eta: float) -> list:
    """CateKV's two budgets per KV head (same page, "CateKV Cache Policy" and
    its benchmark setting): a consistent head keeps its top `budget` entries,
    an adaptive head floor(eta n) of them (eta = 1 keeps them all); never more
    than n."""
    return [min(n, int(np.floor(eta * n))) if a else min(n, int(budget)) for a in adaptive]


def gather_ragged(cache: np.ndarray, idx_list) -> list:
    """Per head, the contiguous copy of its kept rows: [k_h, d_h] each."""
    return [cache[kv, idx] for kv, idx in enumerate(idx_list)]


def window_indices(n: int, n_sink: int, n_keep: int) -> np.ndarray:
    """Rows a sink-plus-recent window reads from a cache of n rows ([Cross] §4.1:
    the StreamingLLM-style comparison policy, which reads as many entries as the
    selection keeps, in place): the first n_sink rows and the most recent
    n_keep - n_sink rows, ascending; every row when n_keep >= n.  The same
    positions for every KV head."""
    if n_keep >= n:
        return np.arange(n, dtype=np.int64)
    if not 0 <= n_sink <= n_keep:
        raise ValueError("need 0 <= n_sink <= n_keep")
    return np.concatenate([np.arange(n_sink), np.arange(n - (n_keep - n_sink), n)]).astype(np.int64)


def gather(cache: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Contiguous copy of the kept rows: [h_kv, k, d_h] from [h_kv, cap, d_h]."""
    return np.stack([cache[kv, idx[kv]] for kv in range(cache.shape[0])])


def select_kv(q_win, k, v, n, n_sink, k_keep, scale=None):
    """Full selection: scores -> float32 -> indices -> gathered K and V."""
    d_h = k.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    s = window_scores(q_win, k, n, scale)
    idx = select_indices(s.astype(np.float32), n, q_win.shape[1], n_sink, k_keep)
    return s, idx, gather(k, idx), gather(v, idx)


# ---------------------------------------------------------------- brute force
def window_scores_loops(q_win, k, n, scale):
    """Pure-Python twin of window_scores for tiny inputs (n, d_h small)."""
    import math
    h_q, w, d_h = q_win.shape
    h_kv = k.shape[0]
    g = h_q // h_kv
    s = [[0.0] * n for _ in range(h_kv)]
    for h in range(h_q):
        kv = h // g
        for i in range(w):
            p = n - w + i
            z = []
            for j in range(p + 1):
                acc = 0.0
                for c in range(d_h):
                    acc += float(q_win[h, i, c]) * float(k[kv, j, c])
                z.append(acc * scale)
            mx = max(z)
            den = sum(math.exp(x - mx) for x in z)
            for j in range(p + 1):
                s[kv][j] += math.exp(z[j] - mx) / den
    return np.array(s)


def select_indices_loops(scores_f32, n, w, n_sink, k_keep):
    """Pure-Python twin of select_indices (selection sort by (-score, j))."""
    h_kv = scores_f32.shape[0]
    if k_keep >= n:
        return np.array([list(range(n))] * h_kv, dtype=np.int32)
    out = []
    for kv in range(h_kv):
        keep = set(range(n_sink)) | set(range(n - w, n))
        pool = list(range(n_sink, n - w))
        for _ in range(k_keep - n_sink - w):
            best = pool[0]
            for j in pool[1:]:
                if float(scores_f32[kv, j]) > float(scores_f32[kv, best]):
                    best = j
            keep.add(best)
            pool.remove(best)
        out.append(sorted(keep))
    return np.array(out, dtype=np.int32)
