"""GPU parity of sd_decode_attn (split-K decode attention) against the float64
oracle's exact attention."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import attention as oatt

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import DEV, TOL, dims_for, rel_l2, to_dev, to_host, workspace  # noqa: E402


def _run(wl, k, v, cap, n_ctx, q, n_splits=0, scale=None):
    dims = dims_for(wl)
    scale = 1.0 / np.sqrt(wl.head_dim) if scale is None else scale
    kd, vd, qd = to_dev(k, wl.dtype), to_dev(v, wl.dtype), to_dev(q)
    out = torch.empty(wl.n_q_heads, wl.head_dim, device=DEV)
    lse = torch.empty(wl.n_q_heads, device=DEV)
    ws = workspace(dims)
    sd.sd_decode_attn(dims, qd, kd, vd, cap, n_ctx, scale, n_splits, out, lse, ws)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


@pytest.mark.parametrize("n_ctx,splits", [(1, 0), (2, 0), (127, 0), (129, 0), (2048, 0),
                                          (2049, 0), (2049, 1), (2049, 3), (2049, 7), (64, 64), (300, 64),
                                          (4099, 17), (300, 128), (4099, 128), (16385, 0),
                                          (16385, 97), (16385, 129), (16385, 200), (4099, 256),
                                          (70001, 0)])
def test_tiny_fp32_matches_oracle(n_ctx, splits):
    wl = synth.TINY
    cap = n_ctx + 5
    k, v = synth.kv_cache(wl, 0, n_ctx, cap)
    q = synth.decode_query(wl, 0)
    out, lse = _run(wl, k, v, cap, n_ctx, q, splits)
    want, want_lse = oatt.attend(q, k, v, n_ctx, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(out, want) <= TOL["f32"]
    assert rel_l2(lse, want_lse) <= TOL["f32"]


@pytest.mark.parametrize("n_ctx", [8193, 32769, 131073])
def test_8b_bf16_matches_oracle(n_ctx):
    # 8B-class shapes at the context lengths of the dense, KV and stacked
    # workloads (rows read = context + the step's own row)
    wl = synth.L8B_DENSE_8K
    k, v = synth.kv_cache(wl, 0, n_ctx, n_ctx)
    q = synth.decode_query(wl, 0)
    out, lse = _run(wl, k, v, n_ctx, n_ctx, q)
    want, want_lse = oatt.attend(q, k, v, n_ctx, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(out, want) <= TOL["bf16"]
    assert rel_l2(lse, want_lse) <= TOL["bf16"]
    # float32 accumulation over exact bf16 inputs is far inside the bf16 bound
    assert rel_l2(out, want) <= 1e-5


def test_special_cases():
    wl = synth.TINY
    n = 777
    k, v = synth.kv_cache(wl, 0, n, n)
    q = synth.decode_query(wl, 0)
    vc = np.full_like(v, 0.375)
    out, _ = _run(wl, k, vc, n, n, q)
    np.testing.assert_allclose(out, 0.375, rtol=1e-6)                    # constant V
    out, lse = _run(wl, k, v, n, 1, q)                                   # one row
    np.testing.assert_allclose(out, v[[0, 0, 1, 1], 0], rtol=1e-6, atol=1e-7)
    out, lse = _run(wl, k, v, n, n, np.zeros_like(q))                    # q = 0
    np.testing.assert_allclose(out, v[[0, 0, 1, 1], :n].mean(1), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(lse, np.log(n), rtol=1e-6)


def test_deterministic_and_split_invariant():
    wl = synth.L8B_DENSE_8K
    n = 20000
    k, v = synth.kv_cache(wl, 3, n, n)
    q = synth.decode_query(wl, 3)
    a, _ = _run(wl, k, v, n, n, q)
    b, _ = _run(wl, k, v, n, n, q)
    assert np.array_equal(a, b)
    c, _ = _run(wl, k, v, n, n, q, n_splits=5)
    assert rel_l2(c, a) <= 1e-6


def test_large_logits_stay_finite():
    # logits near +-80 must not overflow: max subtraction per split and merge
    wl = synth.TINY
    n = 1000
    k, v = synth.kv_cache(wl, 0, n, n)
    q = synth.decode_query(wl, 0) * 40.0
    out, lse = _run(wl, k, v, n, n, q)
    want, want_lse = oatt.attend(q, k, v, n, 1 / np.sqrt(wl.head_dim))
    assert np.all(np.isfinite(out))
    assert rel_l2(out, want) <= 1e-5


# ---- sink-plus-recent window read in place ([Cross] §4.1, §4.4)
from oracle import selection as osel  # noqa: E402


def _run_window(wl, k, v, cap, n_rows, n_sink, n_keep, q, n_splits=0):
    dims = dims_for(wl)
    kd, vd, qd = to_dev(k, wl.dtype), to_dev(v, wl.dtype), to_dev(q)
    out = torch.empty(wl.n_q_heads, wl.head_dim, device=DEV)
    lse = torch.empty(wl.n_q_heads, device=DEV)
    sd.sd_decode_attn_window(dims, qd, kd, vd, cap, n_rows, n_sink, n_keep,
                             1 / np.sqrt(wl.head_dim), n_splits, out, lse, workspace(dims))
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


@pytest.mark.parametrize("n_rows,n_sink,n_keep,splits", [(2049, 4, 614, 0), (2049, 0, 614, 0),
                                                         (2049, 614, 614, 0), (500, 4, 600, 0),
                                                         (4099, 4, 1229, 7), (300, 4, 5, 0)])
def test_window_tiny_fp32_matches_oracle(n_rows, n_sink, n_keep, splits):
    wl = synth.TINY
    cap = n_rows + 3
    k, v = synth.kv_cache(wl, 1, n_rows, cap)
    q = synth.decode_query(wl, 1)
    out, lse = _run_window(wl, k, v, cap, n_rows, n_sink, n_keep, q, splits)
    idx = osel.window_indices(n_rows, n_sink, n_keep)
    want, want_lse = oatt.attend(q, k[:, idx], v[:, idx], len(idx), 1 / np.sqrt(wl.head_dim))
    assert rel_l2(out, want) <= TOL["f32"]
    assert rel_l2(lse, want_lse) <= TOL["f32"]


def test_window_8b_bf16_30pct_at_32k():
    wl = synth.L8B_KV_32K
    n = 32769
    k, v = synth.kv_cache(wl, 0, n, n)
    q = synth.decode_query(wl, 0)
    keep = int(0.3 * n)
    out, lse = _run_window(wl, k, v, n, n, 4, keep, q)
    idx = osel.window_indices(n, 4, keep)
    want, want_lse = oatt.attend(q, k[:, idx], v[:, idx], len(idx), 1 / np.sqrt(wl.head_dim))
    assert rel_l2(out, want) <= 1e-5 and rel_l2(lse, want_lse) <= 1e-5


# ---- deliberately plain dense comparison paths ([Cross] §4.4)
@pytest.mark.parametrize("path", ["masked", "fused"])
@pytest.mark.parametrize("n_ctx,extra", [(1, 0), (777, 5), (2049, 300), (4100, 0)])
def test_baselines_tiny_fp32_match_oracle(path, n_ctx, extra):
    wl = synth.TINY
    cap = n_ctx + extra
    k, v = synth.kv_cache(wl, 2, n_ctx, cap)
    k[:, n_ctx:] = np.nan  # rows past n_ctx are allocated but hold anything
    v[:, n_ctx:] = np.nan
    q = synth.decode_query(wl, 2)
    dims = dims_for(wl)
    code = {"masked": sd.SD_ATTN_MASKED, "fused": sd.SD_ATTN_FUSED}[path]
    out = torch.empty(wl.n_q_heads, wl.head_dim, device=DEV)
    lse = torch.empty(wl.n_q_heads, device=DEV)
    ws = workspace(dims, cap)
    sd.sd_decode_attn_baseline(dims, to_dev(q), to_dev(k), to_dev(v), cap, n_ctx,
                               1 / np.sqrt(wl.head_dim), code, out, lse, ws)
    torch.cuda.synchronize()
    want, want_lse = oatt.attend(q, k, v, n_ctx, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(to_host(out), want) <= TOL["f32"]
    assert rel_l2(to_host(lse), want_lse) <= TOL["f32"]


@pytest.mark.parametrize("path", ["masked", "fused"])
def test_baselines_8b_bf16_match_oracle(path):
    wl = synth.L8B_DENSE_8K
    n, cap = 8193, 8300
    k, v = synth.kv_cache(wl, 1, n, cap)
    q = synth.decode_query(wl, 1)
    dims = dims_for(wl)
    code = {"masked": sd.SD_ATTN_MASKED, "fused": sd.SD_ATTN_FUSED}[path]
    out = torch.empty(wl.n_q_heads, wl.head_dim, device=DEV)
    sd.sd_decode_attn_baseline(dims, to_dev(q), to_dev(k, "bf16"), to_dev(v, "bf16"), cap, n,
                               1 / np.sqrt(wl.head_dim), code, out, None, workspace(dims, cap))
    torch.cuda.synchronize()
    want, _ = oatt.attend(q, k, v, n, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(to_host(out), want) <= 1e-5


@pytest.mark.parametrize("h_q,h_kv", [(8, 8), (64, 8)])
@pytest.mark.parametrize("dtype,dh", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("n_ctx,splits", [(4099, 0), (20001, 256), (20001, 129), (20001, 8)])
def test_query_group_sizes_match_oracle(h_q, h_kv, dtype, dh, n_ctx, splits):
    # one and eight query heads per KV head (the kernel's other group
    # instances), up to the largest split count and the widest merge, and
    # 2501-row chunks (the three-buffer instances)
    wl = dataclasses.replace(synth.L8B_DENSE_8K, name=f"attn-g{h_q // h_kv}-{dtype}", wid=6,
                             n_q_heads=h_q, n_kv_heads=h_kv, head_dim=dh, dtype=dtype)
    k, v = synth.kv_cache(wl, 0, n_ctx, n_ctx + 3)
    q = synth.decode_query(wl, 0)
    out, lse = _run(wl, k, v, n_ctx + 3, n_ctx, q, splits)
    want, want_lse = oatt.attend(q, k, v, n_ctx, 1 / np.sqrt(dh))
    tol = TOL["bf16"] if dtype == "bf16" else TOL["f32"]
    assert rel_l2(out, want) <= tol
    assert rel_l2(lse, want_lse) <= tol
