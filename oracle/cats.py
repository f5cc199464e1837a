"""Oracle: CATS-style sparse SwiGLU MLP (test infrastructure only).

[SATS] keeps the CATS runtime masking and changes only how its per-layer
threshold is calibrated.  The runtime rule: compute the gate projection,
apply SiLU, and drop every channel whose post-gate activation magnitude is
below the layer's threshold t; only the kept channels' up-projection rows and
down-projection columns then contribute.  CATS itself picks t as a percentile
of the empirical distribution of |post-gate activation| on calibration data.

Exact for a given mask: the sparse MLP equals the dense SwiGLU with dropped
channels zeroed, so the oracle computes it masked-dense

    g = W_gate x,  a = g * sigmoid(g),  u = W_up x
    y = W_down (mask * a * u)

and gathering only the kept channels is the kernel's way of reaching it.

Readings:
* keep channel i iff |a_i| > t (strict); t < 0 means dense.  The [SATS] text
  drops values "below" t, which would keep |a| == t; the strict form is the
  one the hot path states, and |a| == t is then dropped.
* the mask is decided on float32 |a| (the kernel's precision; the pages fix
  none), so both sides agree when handed the same float32 activations.
* calibration: sort the float32 |a| calibration values ascending as v; for a
  target sparsity s over N values take k = round(s N) and t = v[k-1]
  (t = -1, i.e. dense, when k = 0).  With no ties exactly k values then satisfy
  |a| <= t, so the realized sparsity on the calibration set is k / N.

Pins (tests/test_oracle_cats.py): t < 0 and t = 0 reproduce the dense SwiGLU
bit for bit; the gathered form (loop over kept channels) equals the
masked-dense form; SiLU matches its closed form at special points; the
calibrated threshold realizes exactly k of N on tie-free data.
"""

from __future__ import annotations

import numpy as np


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def gate_act(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    """a = SiLU(W_gate x) in float64: [d_ff]."""
    return silu(w_gate.astype(np.float64) @ x.astype(np.float64))


def cats_mask(act_f32: np.ndarray, t: float) -> np.ndarray:
    """Keep mask from float32 activations: |a| > t, or all when t < 0."""
    act_f32 = np.asarray(act_f32)
    if act_f32.dtype != np.float32:
        raise TypeError("the mask is decided on float32 activations")
    t32 = np.float32(t)
    if t32 < 0:
        return np.ones(act_f32.shape, dtype=bool)
    return np.abs(act_f32) > t32


def kept_indices(mask: np.ndarray) -> np.ndarray:
    """Ascending kept channel list (int32)."""
    return np.flatnonzero(mask).astype(np.int32)


def mlp_masked(x, w_gate, w_up, w_down_t, mask, act=None):
    """y = W_down (mask * a * (W_up x)); W_down is stored transposed [d_ff, d]."""
    x64 = np.asarray(x, dtype=np.float64)
    a = gate_act(x64, w_gate) if act is None else np.asarray(act, dtype=np.float64)
    u = w_up.astype(np.float64) @ x64
    hmid = np.where(mask, a * u, 0.0)
    return w_down_t.astype(np.float64).T @ hmid


def cats_mlp(x, w_gate, w_up, w_down_t, t):
    """Full CATS MLP with the mask taken on the float32 rounding of a.

    Returns (y, a, mask, idx)."""
    a = gate_act(x, w_gate)
    mask = cats_mask(a.astype(np.float32), t)
    y = mlp_masked(x, w_gate, w_up, w_down_t, mask, act=a)
    return y, a, mask, kept_indices(mask)


def dense_swiglu(x, w_gate, w_up, w_down_t):
    """Dense SwiGLU in the same operation order as mlp_masked (no mask)."""
    x64 = np.asarray(x, dtype=np.float64)
    a = silu(w_gate.astype(np.float64) @ x64)
    u = w_up.astype(np.float64) @ x64
    return w_down_t.astype(np.float64).T @ (a * u)


def mlp_gathered_loops(x, w_gate, w_up, w_down_t, idx):
    """Gathered twin: loop over the kept channels only (small inputs)."""
    x64 = np.asarray(x, dtype=np.float64)
    y = np.zeros(w_down_t.shape[1])
    for i in idx:
        g = float(w_gate[i].astype(np.float64) @ x64)
        a = g / (1.0 + np.exp(-g))
        u = float(w_up[i].astype(np.float64) @ x64)
        y += a * u * w_down_t[i].astype(np.float64)
    return y


def calibrate_threshold(abs_act_f32: np.ndarray, sparsity: float) -> float:
    """Per-layer threshold from calibration magnitudes (float32 values)."""
    v = np.sort(np.asarray(abs_act_f32, dtype=np.float32).ravel())
    k = int(round(sparsity * v.size))
    if k <= 0:
        return -1.0
    return float(v[k - 1])
