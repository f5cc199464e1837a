"""Oracle: one decoder layer and a full decode step (test infrastructure only).

[Cross] times Llama-family decoders (§4.1) at batch size one; the layer's
exact form is not on the pages, so the reading here is the standard pre-norm
Llama layer without biases:

    x  = RMSNorm(h) * attn_norm
    q, k, v = W_qkv x                      (fused rows: q | k | v)
    q, k = RoPE(q, pos), RoPE(k, pos)       (rotate-half pairs (i, i + d_h/2))
    append round(k), round(v) at row n of the full cache and, if the layer
        has a gathered buffer, at its row n_sel too   ([Cross] §3.2, §4.1)
    o  = attention over rows 0..n of the full cache   (dense mode)
         or rows 0..n_sel of the gathered buffer      (KV mode)
         or the sinks plus the most recent rows of the full cache, read in
         place (window mode, [Cross] §4.1, §4.4)
    h += W_o o
    x  = RMSNorm(h) * mlp_norm
    h += CATS-MLP(x, t)  (dense when the MLP branch is off or t < 0)

pos is the absolute position of the new token (= the full cache length n
before the append).  RoPE uses theta (500000 for Llama-3.x; theta <= 0 turns
it off) with no frequency scaling.  Cached keys and window queries of the
synthetic workloads are taken as already rotated.  The appended key and value
are rounded to the cache element type: float32, or bfloat16 by
round-to-nearest-even directly from float64.

Pins (tests/test_oracle_step.py): RoPE at position 0 is the identity, it
preserves norms, and q(m).k(m') depends only on m - m'; RMSNorm of a
constant vector has a closed form; bfloat16 rounding matches torch's
float32 -> bfloat16 conversion on float32 inputs; a step with the KV branch at
keep ratio 1 and the MLP branch at t < 0 is bit-identical to the dense step.
"""

from __future__ import annotations

import numpy as np

from . import attention, cats


def rmsnorm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x) + eps) * np.asarray(weight, dtype=np.float64)


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate-half RoPE of x [heads, d_h] at absolute position pos."""
    x = np.asarray(x, dtype=np.float64)
    if theta <= 0:
        return x.copy()
    d_h = x.shape[-1]
    half = d_h // 2
    inv_freq = theta ** (-(2.0 * np.arange(half)) / d_h)
    ang = float(pos) * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); float64 out.

    bfloat16 keeps 8 significant bits and float32's exponent range (normal
    values from 2**-126, subnormal spacing 2**-133).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    e = np.floor(np.log2(np.abs(x[nz])))
    # np.log2 can land one off near powers of two; fix the exponent exactly.
    e = np.where(2.0 ** e > np.abs(x[nz]), e - 1, e)
    e = np.where(2.0 ** (e + 1) <= np.abs(x[nz]), e + 1, e)
    ulp = 2.0 ** np.maximum(e - 7, -133)
    out[nz] = np.round(x[nz] / ulp) * ulp  # np.round: half to even
    big = np.abs(out) > 3.3895313892515355e38
    out[big] = np.sign(out[big]) * np.inf
    return out


def round_to_cache(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "bf16":
        return round_to_bf16(x)
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(kv_dtype)


class Layer:
    """One layer's weights and caches as float64 arrays (values exactly those
    of the bf16 / fp32 tensors the HIP path holds)."""

    def __init__(self, attn_norm, w_qkv, w_o, mlp_norm, w_gate, w_up, w_down_t,
                 threshold, k_full, v_full, n, k_sel=None, v_sel=None, n_sel=0,
                 n_sel_heads=None):
        self.attn_norm = np.asarray(attn_norm, dtype=np.float64)
        self.w_qkv = np.asarray(w_qkv, dtype=np.float64)
        self.w_o = np.asarray(w_o, dtype=np.float64)
        self.mlp_norm = np.asarray(mlp_norm, dtype=np.float64)
        self.w_gate = np.asarray(w_gate, dtype=np.float64)
        self.w_up = np.asarray(w_up, dtype=np.float64)
        self.w_down_t = np.asarray(w_down_t, dtype=np.float64)
        self.threshold = float(threshold)
        self.k_full = np.array(k_full, dtype=np.float64)
        self.v_full = np.array(v_full, dtype=np.float64)
        self.n = int(n)
        self.k_sel = None if k_sel is None else np.array(k_sel, dtype=np.float64)
        self.v_sel = None if v_sel is None else np.array(v_sel, dtype=np.float64)
        self.n_sel = int(n_sel)
        # ragged budgets: valid gathered rows per KV head (n_sel is then unused)
        self.n_sel_heads = None if n_sel_heads is None else [int(x) for x in n_sel_heads]


def decode_layer(layer: Layer, h: np.ndarray, pos: int, *, n_q_heads: int,
                 n_kv_heads: int, head_dim: int, kv_dtype: str, kv_sparse: bool,
                 mlp_sparse: bool, eps: float = 1e-5, theta: float = 500000.0,
                 mask_override=None, trace=None, kv_window=None) -> np.ndarray:
    """One layer; appends to layer's caches in place and returns the new h.
    kv_window = (n_sink, n_keep) attends over selection.window_indices of the
    full cache instead (after the append)."""
    h = np.asarray(h, dtype=np.float64).copy()
    qd = n_q_heads * head_dim
    kd = n_kv_heads * head_dim
    x = rmsnorm(h, layer.attn_norm, eps)
    qkv = layer.w_qkv @ x
    q = rope(qkv[:qd].reshape(n_q_heads, head_dim), pos, theta)
    k = rope(qkv[qd:qd + kd].reshape(n_kv_heads, head_dim), pos, theta)
    v = qkv[qd + kd:qd + 2 * kd].reshape(n_kv_heads, head_dim)
    k_r = round_to_cache(k, kv_dtype)
    v_r = round_to_cache(v, kv_dtype)
    layer.k_full[:, layer.n] = k_r
    layer.v_full[:, layer.n] = v_r
    layer.n += 1
    if layer.k_sel is not None:
        if layer.n_sel_heads is not None:  # ragged: each KV head appends at its own row
            for kv in range(n_kv_heads):
                layer.k_sel[kv, layer.n_sel_heads[kv]] = k_r[kv]
                layer.v_sel[kv, layer.n_sel_heads[kv]] = v_r[kv]
                layer.n_sel_heads[kv] += 1
        else:
            layer.k_sel[:, layer.n_sel] = k_r
            layer.v_sel[:, layer.n_sel] = v_r
            layer.n_sel += 1
    scale = 1.0 / np.sqrt(head_dim)
    if kv_sparse and layer.n_sel_heads is not None:
        if kv_window is not None:
            raise ValueError("ragged budgets and the window are separate policies")
        o, _ = attention.attend_ragged(q, layer.k_sel, layer.v_sel, layer.n_sel_heads, scale)
    elif kv_window is not None:
        from . import selection
        idx = selection.window_indices(layer.n, kv_window[0], kv_window[1])
        o, _ = attention.attend(q, layer.k_full[:, idx], layer.v_full[:, idx], len(idx), scale)
    elif kv_sparse:
        if layer.k_sel is None:
            raise ValueError("KV-sparse mode needs a gathered buffer")
        o, _ = attention.attend(q, layer.k_sel, layer.v_sel, layer.n_sel, scale)
    else:
        o, _ = attention.attend(q, layer.k_full, layer.v_full, layer.n, scale)
    h = h + layer.w_o @ o.reshape(-1)
    x2 = rmsnorm(h, layer.mlp_norm, eps)
    a = cats.gate_act(x2, layer.w_gate)
    t = layer.threshold if mlp_sparse else -1.0
    if mask_override is not None:
        mask = np.asarray(mask_override, dtype=bool)
    else:
        mask = cats.cats_mask(a.astype(np.float32), t)
    y = cats.mlp_masked(x2, layer.w_gate, layer.w_up, layer.w_down_t, mask, act=a)
    if trace is not None:
        trace.append(dict(q=q, k=k, v=v, attn=o, act=a, mask=mask, y=y))
    return h + y


def decode_step(layers, h, pos, *, kv_sparse, mlp_sparse, masks=None, trace=None,
                kv_window=None, **dims):
    """All layers in order; returns the new hidden state."""
    for li, layer in enumerate(layers):
        m = None if masks is None else masks[li]
        h = decode_layer(layer, h, pos, kv_sparse=kv_sparse, mlp_sparse=mlp_sparse,
                         mask_override=m, trace=trace, kv_window=kv_window, **dims)
    return h
