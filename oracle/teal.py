"""Oracle: TEAL-style sparsity on all seven projections (test infrastructure only).

"Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding" takes
its projection branch from TEAL (§3.2 "Sparse Branches", §4.1 "Setup"): every
one of a layer's seven projections -- W_q, W_k, W_v, W_o and the three
feed-forward matrices -- keeps only the input activation channels whose
magnitude clears a calibrated threshold, and loads only the weight columns of
those channels.  For one projection y = W x that is

    keep j  iff  |x_j| > t   (t < 0: keep all)
    y = W (mask * x)  =  sum over kept j of x_j W[:, j]

Exact for a given mask, so the oracle computes it masked-dense; reading only
the kept columns (rows of the stored transpose) is the kernel's way of
reaching the same sum.

Readings:
* inputs shared by several projections share one mask: W_q, W_k, W_v read
  the attention-norm output, W_gate and W_up the MLP-norm output.  A layer
  therefore has four thresholds: attention input, O input (the attention
  output), MLP input, and down input (SiLU(W_gate x) * (W_up x));
* keep iff |x_j| > t, strict, with the decision on float32 values (the
  kernel's precision), as for the CATS mask;
* the feed-forward block stays SwiGLU with no CATS gate mask: the gate and
  up projections see the sparsified MLP input, the down projection its own
  sparsified input;
* thresholds: the same percentile rule as CATS calibration (cats.calibrate_
  threshold) applied to each input's float32 magnitudes.

Pins (tests/test_oracle_teal.py): t < 0 reproduces the dense projection and
the dense layer bit for bit; the loop over kept channels equals the
masked-dense form; an all-drop mask gives zero; the realised keep fraction
of a calibrated threshold on tie-free data is exact; a closed-form
two-channel case.
"""

from __future__ import annotations

import numpy as np

from . import attention, cats
from .step import rmsnorm, rope, round_to_cache

# index of each threshold / mask in a layer's four
ATTN_IN, O_IN, MLP_IN, DOWN_IN = 0, 1, 2, 3


def teal_mask(x_f32: np.ndarray, t: float) -> np.ndarray:
    """Keep mask from float32 inputs: |x| > t, or all when t < 0."""
    x_f32 = np.asarray(x_f32)
    if x_f32.dtype != np.float32:
        raise TypeError("the mask is decided on float32 inputs")
    t32 = np.float32(t)
    if t32 < 0:
        return np.ones(x_f32.shape, dtype=bool)
    return np.abs(x_f32) > t32


def linear_masked(w: np.ndarray, x: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """y = W (mask * x) in float64; W is [out, in]."""
    x64 = np.where(np.asarray(mask, dtype=bool), np.asarray(x, dtype=np.float64), 0.0)
    return np.asarray(w, dtype=np.float64) @ x64


def linear_gathered_loops(w_t: np.ndarray, x: np.ndarray, idx) -> np.ndarray:
    """Gathered twin over the stored transpose w_t [in, out]: sum of x_j w_t[j]
    over the kept inputs only (small inputs)."""
    x64 = np.asarray(x, dtype=np.float64)
    y = np.zeros(np.asarray(w_t).shape[1])
    for j in idx:
        y += x64[j] * np.asarray(w_t[j], dtype=np.float64)
    return y


def teal_linear(w, x, t):
    """One TEAL projection with the mask decided on the float32 rounding of x.
    Returns (y, mask, idx)."""
    mask = teal_mask(np.asarray(x, dtype=np.float64).astype(np.float32), t)
    return linear_masked(w, x, mask), mask, np.flatnonzero(mask).astype(np.int32)


def teal_layer(layer, h, pos, thresholds, *, n_q_heads, n_kv_heads, head_dim, kv_dtype,
               kv_sparse, eps=1e-5, theta=500000.0, masks=None, trace=None):
    """One decode layer (step.Layer) with all seven projections TEAL-sparse.

    thresholds: (t_attn_in, t_o_in, t_mlp_in, t_down_in); masks: optional four
    boolean arrays that replace the decisions (to test a kernel's own masks).
    Appends to the layer's caches in place and returns the new h."""
    h = np.asarray(h, dtype=np.float64).copy()
    qd = n_q_heads * head_dim
    kd = n_kv_heads * head_dim

    def mask_of(k, x):
        if masks is not None:
            return np.asarray(masks[k], dtype=bool)
        return teal_mask(x.astype(np.float32), thresholds[k])

    x = rmsnorm(h, layer.attn_norm, eps)
    m_a = mask_of(ATTN_IN, x)
    qkv = linear_masked(layer.w_qkv, x, m_a)
    q = rope(qkv[:qd].reshape(n_q_heads, head_dim), pos, theta)
    k = rope(qkv[qd:qd + kd].reshape(n_kv_heads, head_dim), pos, theta)
    v = qkv[qd + kd:qd + 2 * kd].reshape(n_kv_heads, head_dim)
    k_r = round_to_cache(k, kv_dtype)
    v_r = round_to_cache(v, kv_dtype)
    layer.k_full[:, layer.n] = k_r
    layer.v_full[:, layer.n] = v_r
    layer.n += 1
    ragged = getattr(layer, "n_sel_heads", None) is not None
    if layer.k_sel is not None:
        if ragged:
            for kv in range(n_kv_heads):
                layer.k_sel[kv, layer.n_sel_heads[kv]] = k_r[kv]
                layer.v_sel[kv, layer.n_sel_heads[kv]] = v_r[kv]
                layer.n_sel_heads[kv] += 1
        else:
            layer.k_sel[:, layer.n_sel] = k_r
            layer.v_sel[:, layer.n_sel] = v_r
            layer.n_sel += 1
    scale = 1.0 / np.sqrt(head_dim)
    if kv_sparse and ragged:
        o, _ = attention.attend_ragged(q, layer.k_sel, layer.v_sel, layer.n_sel_heads, scale)
    elif kv_sparse:
        o, _ = attention.attend(q, layer.k_sel, layer.v_sel, layer.n_sel, scale)
    else:
        o, _ = attention.attend(q, layer.k_full, layer.v_full, layer.n, scale)
    o = o.reshape(-1)
    m_o = mask_of(O_IN, o)
    h = h + linear_masked(layer.w_o, o, m_o)
    x2 = rmsnorm(h, layer.mlp_norm, eps)
    m_m = mask_of(MLP_IN, x2)
    g = linear_masked(layer.w_gate, x2, m_m)
    u = linear_masked(layer.w_up, x2, m_m)
    hmid = cats.silu(g) * u
    m_d = mask_of(DOWN_IN, hmid)
    y = linear_masked(np.asarray(layer.w_down_t, dtype=np.float64).T, hmid, m_d)
    if trace is not None:
        trace.append(dict(x=x, q=q, k=k, v=v, attn=o, x2=x2, hmid=hmid,
                          masks=(m_a, m_o, m_m, m_d), y=y))
    return h + y


def teal_step(layers, h, pos, thresholds, *, kv_sparse, masks=None, trace=None, **dims):
    """All layers in order; thresholds[l] and masks[l] per layer."""
    for li, layer in enumerate(layers):
        m = None if masks is None else masks[li]
        h = teal_layer(layer, h, pos, thresholds[li], kv_sparse=kv_sparse, masks=m,
                       trace=trace, **dims)
    return h
