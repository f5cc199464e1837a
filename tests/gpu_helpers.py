"""Helpers for the GPU parity tests: device copies of seeded inputs, the
relative-L2 metric and tolerances, workspace allocation, and oracle-side
threshold choice.  Nothing here computes a GPU-side expected value."""

from __future__ import annotations

import copy

import numpy as np
import torch

import kv_cache_activation_amd as sd
import synth
from oracle import step as ostep

DEV = torch.device("cuda:0")

# Relative L2 tolerance per input element type: bf16 inputs with float32
# accumulation, or float32 throughout.
TOL = {"bf16": 3e-3, "f32": 1e-5}


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def to_dev(a: np.ndarray, dtype: str = "f32") -> torch.Tensor:
    """float32 array (bfloat16-representable when dtype == 'bf16') -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: the values are already bfloat16
    return t.to(DEV)


def teal_dev(w_out_in: np.ndarray, dtype: str = "f32") -> torch.Tensor:
    """A projection W [d_out, d_in] on the device in the column-block layout
    the TEAL projections read ([ceil(d_out / 128)][d_in][128])."""
    from synth import device as sdev
    return sdev.teal_blocked(to_dev(np.ascontiguousarray(w_out_in), dtype))


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def dims_for(wl: synth.Workload, theta: float = 500000.0):
    code = sd.SD_BF16 if wl.dtype == "bf16" else sd.SD_F32
    return sd.make_dims(wl.d_model, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff, code, code,
                        1e-5, theta)


def workspace(dims, rows: int = 0, window: int = 0) -> torch.Tensor:
    return torch.empty(sd.sd_workspace_bytes(dims, rows, window), dtype=torch.uint8, device=DEV)


def midpoint_threshold(act: np.ndarray, sparsity: float) -> float:
    """A threshold halfway between the k-th and (k+1)-th smallest float32 |a|
    (k = round(sparsity * N)): exactly k channels fall below it, and no
    channel sits within half a gap of it, so rounding differences of order
    1e-6 cannot flip a channel."""
    v = np.sort(np.abs(np.asarray(act).astype(np.float32)))
    k = int(np.floor(sparsity * v.size + 0.5))
    if k <= 0:
        return -1.0
    return float((np.float64(v[k - 1]) + np.float64(v[k])) / 2)


def oracle_thresholds(layers, h, pos, sparsity, kv_sparse, odims, kv_window=None):
    """Per-layer midpoint thresholds from the oracle's own activations, layer by
    layer (a layer's gate input does not depend on its own threshold).  The
    oracle layers are left untouched; returns the list of thresholds."""
    work = copy.deepcopy(layers)
    ts = []
    hh = np.asarray(h, dtype=np.float64)
    for layer in work:
        tr = []
        probe = copy.deepcopy(layer)
        ostep.decode_layer(probe, hh, pos, kv_sparse=kv_sparse, mlp_sparse=False, trace=tr,
                           kv_window=kv_window, **odims)
        t = midpoint_threshold(tr[0]["act"], sparsity)
        layer.threshold = t
        hh = ostep.decode_layer(layer, hh, pos, kv_sparse=kv_sparse, mlp_sparse=True,
                                kv_window=kv_window, **odims)
        ts.append(t)
    return ts
