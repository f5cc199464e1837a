"""Seeded synthetic inputs shaped like the pages' decode workloads.

This module holds input recipes only -- random draws, rounding of the draws to
bfloat16-representable values, and the shapes of the five workloads -- and
none of the arithmetic of the method.  Tests hand the same arrays to the
float64 oracle and to the HIP library; the benchmark uses the same recipes
(drawn on the device at sizes the host cannot hold cheaply).

Recipes (the pages use real text and trained weights, which are not here):
* weights ~ N(0, 0.02^2), rounded to the weight type; norm vectors are ones;
* cached K, V ~ N(0, 1), multiplied per (KV head, channel) by scales drawn
  from LogNormal(0, 0.5) for the 8B-class workloads (outlier channels);
* window queries and decode queries ~ N(0, 1); hidden state ~ N(0, 1);
* adaptive heads (CateKV's head classes, which the pages obtain offline from
  reference data): round(ratio * n_kv_heads * n_layers) adaptive KV heads in
  all, each layer holding the floor or the ceiling of the per-layer mean,
  layers and heads picked by seeded permutations;
* planted keys (retrieval stand-in): 64 positions drawn without replacement
  from the non-forced range, shared by all KV heads; the key at each is
  4 sqrt(d_h) times the unit vector along the sum of that KV head's window
  queries, so its logits sit near 4 standard deviations above the background.

Seeds: numpy.random.SeedSequence([0, workload, layer, tensor]) with PCG64.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

# tensor ids for the seed sequence
T_QKV, T_O, T_GATE, T_UP, T_DOWN, T_K, T_V, T_KSCALE, T_VSCALE = range(9)
T_QWIN, T_Q, T_H, T_PLANT, T_CAL, T_PARTIALS, T_GATE_IN, T_ADAPT = range(9, 17)


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    dtype: str            # "f32" or "bf16" for weights and caches
    n_layers: int
    n_ctx: int
    channel_scale: bool   # LogNormal(0, 0.5) per (KV head, channel) on K and V
    window: int = 32
    n_sink: int = 4
    keep_ratio: float = 1.0
    sparsity: tuple = ()  # CATS target gate sparsities
    n_planted: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def k_keep(self) -> int:
        return int(np.floor(self.keep_ratio * self.n_ctx))

    @property
    def qkv_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def with_ctx(self, n_ctx: int) -> "Workload":
        return replace(self, n_ctx=n_ctx)


TINY = Workload("tiny-fp32-1layer-ctx2048", 0, 256, 4, 2, 64, 688, "f32", 1, 2048,
                False, keep_ratio=0.25, sparsity=(0.5,),
                notes="CATS threshold from the step's own gate vector")
L8B_DENSE_8K = Workload("8b-layer-bf16-dense-ctx8192", 1, 4096, 32, 8, 128, 14336,
                        "bf16", 1, 8192, True)
L8B_KV_32K = Workload("8b-layer-bf16-kv16-ctx32768", 2, 4096, 32, 8, 128, 14336,
                      "bf16", 1, 32768, True, keep_ratio=0.16, n_planted=64)
L8B_CATS_4K = Workload("8b-layer-bf16-cats-ctx4096", 3, 4096, 32, 8, 128, 14336,
                       "bf16", 1, 4096, True, sparsity=(0.5, 0.7))
STACK32_128K = Workload("8b-32layer-bf16-both-ctx131072", 4, 4096, 32, 8, 128, 14336,
                        "bf16", 32, 131072, True, keep_ratio=0.10, sparsity=(0.5,))
WORKLOADS = (TINY, L8B_DENSE_8K, L8B_KV_32K, L8B_CATS_4K, STACK32_128K)
SWEEP_CTX = (2048, 8192, 32768, 65536, 131072)


def rng(wid: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, wid, layer, tensor])))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bfloat16-representable")
    return (u >> 16).astype(np.uint16)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32)
    return to_bf16_values(x) if dtype == "bf16" else x


def layer_weights(wl: Workload, layer: int) -> dict:
    """float32 arrays whose values are exactly those of the stored weights."""
    d, f = wl.d_model, wl.d_ff
    hd = wl.n_q_heads * wl.head_dim

    def w(tid, shape):
        return _cast(rng(wl.wid, layer, tid).standard_normal(shape, dtype=np.float32) * 0.02,
                     wl.dtype)

    return dict(
        attn_norm=np.ones(d, np.float32),
        w_qkv=w(T_QKV, (wl.qkv_out, d)),
        w_o=w(T_O, (d, hd)),
        mlp_norm=np.ones(d, np.float32),
        w_gate=w(T_GATE, (f, d)),
        w_up=w(T_UP, (f, d)),
        w_down_t=w(T_DOWN, (f, d)),
    )


def kv_cache(wl: Workload, layer: int, n: int, cap: int) -> tuple[np.ndarray, np.ndarray]:
    """K, V [h_kv, cap, d_h]; rows >= n are zero."""
    shape = (wl.n_kv_heads, cap, wl.head_dim)
    k = np.zeros(shape, np.float32)
    v = np.zeros(shape, np.float32)
    k[:, :n] = rng(wl.wid, layer, T_K).standard_normal((wl.n_kv_heads, n, wl.head_dim),
                                                         dtype=np.float32)
    v[:, :n] = rng(wl.wid, layer, T_V).standard_normal((wl.n_kv_heads, n, wl.head_dim),
                                                         dtype=np.float32)
    if wl.channel_scale:
        sk = rng(wl.wid, layer, T_KSCALE).lognormal(0.0, 0.5, (wl.n_kv_heads, 1, wl.head_dim))
        sv = rng(wl.wid, layer, T_VSCALE).lognormal(0.0, 0.5, (wl.n_kv_heads, 1, wl.head_dim))
        k[:, :n] *= sk.astype(np.float32)
        v[:, :n] *= sv.astype(np.float32)
    return _cast(k, wl.dtype), _cast(v, wl.dtype)


def window_queries(wl: Workload, layer: int) -> np.ndarray:
    return rng(wl.wid, layer, T_QWIN).standard_normal(
        (wl.n_q_heads, wl.window, wl.head_dim), dtype=np.float32)


def plant_keys(wl: Workload, layer: int, k: np.ndarray, n: int, q_win: np.ndarray,
               n_planted: int | None = None) -> np.ndarray:
    """Overwrite planted positions of k in place; returns the sorted positions."""
    n_planted = wl.n_planted if n_planted is None else n_planted
    if n_planted == 0:
        return np.zeros(0, np.int64)
    lo, hi = wl.n_sink, n - wl.window
    pos = np.sort(rng(wl.wid, layer, T_PLANT).choice(np.arange(lo, hi), n_planted,
                                                     replace=False))
    g = wl.n_q_heads // wl.n_kv_heads
    for kv in range(wl.n_kv_heads):
        s = q_win[kv * g:(kv + 1) * g].astype(np.float64).sum(axis=(0, 1))
        u = s / np.linalg.norm(s)
        key = (4.0 * np.sqrt(wl.head_dim) * u).astype(np.float32)
        k[kv, pos] = _cast(key, wl.dtype)
    return pos


def decode_query(wl: Workload, layer: int) -> np.ndarray:
    return rng(wl.wid, layer, T_Q).standard_normal((wl.n_q_heads, wl.head_dim),
                                                   dtype=np.float32)


def hidden(wl: Workload, draw: int = 0) -> np.ndarray:
    return rng(wl.wid, 1000 + draw, T_H).standard_normal(wl.d_model, dtype=np.float32)


def calibration_states(wl: Workload, layer: int, n_states: int = 256) -> np.ndarray:
    return rng(wl.wid, layer, T_CAL).standard_normal((n_states, wl.d_model),
                                                     dtype=np.float32)


def catekv_adaptive(wl: Workload, n_layers: int, ratio: float = 0.4) -> list:
    """Per layer, which KV heads are adaptive (True) or consistent (False)."""
    h = wl.n_kv_heads
    total = int(np.floor(ratio * h * n_layers + 0.5))
    base, extra = divmod(total, n_layers)
    r = rng(wl.wid, 0, T_ADAPT)
    more = set(r.permutation(n_layers)[:extra].tolist())
    out = []
    for li in range(n_layers):
        k = base + (1 if li in more else 0)
        heads = set(rng(wl.wid, li, T_ADAPT).permutation(h)[:k].tolist())
        out.append([j in heads for j in range(h)])
    return out
