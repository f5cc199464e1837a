"""Pins of the oracle's decoder layer: RMSNorm, RoPE, bfloat16 rounding and the
composed step (Llama-style pre-norm layer; modes of "Where Activation Sparsity
and KV-Cache Sparsity Cross in LLM Decoding", §3.2 and §5.3)."""

import copy

import numpy as np
import pytest
import torch

from oracle import selection, step


def test_rmsnorm_constant_vector_closed_form():
    x = np.full(64, 3.0)
    np.testing.assert_allclose(step.rmsnorm(x, np.ones(64), 1e-5), 3.0 / np.sqrt(9.0 + 1e-5))


def test_rmsnorm_matches_torch():
    x = np.random.default_rng(0).standard_normal(96)
    w = np.random.default_rng(1).standard_normal(96)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), 1e-5)
    np.testing.assert_allclose(step.rmsnorm(x, w, 1e-5), want.numpy(), rtol=1e-14)


def test_rope_properties():
    r = np.random.default_rng(2)
    q = r.standard_normal((3, 64))
    k = r.standard_normal((3, 64))
    assert np.array_equal(step.rope(q, 0, 5e5), q)
    np.testing.assert_allclose(np.linalg.norm(step.rope(q, 12345, 5e5), axis=1),
                               np.linalg.norm(q, axis=1), rtol=1e-13)
    a = (step.rope(q, 100, 5e5) * step.rope(k, 37, 5e5)).sum(1)
    b = (step.rope(q, 1100, 5e5) * step.rope(k, 1037, 5e5)).sum(1)
    np.testing.assert_allclose(a, b, rtol=1e-9)


def test_rope_matches_complex_rotation():
    # independent form: pair (x_i, x_{i+d/2}) as a complex number times e^{i pos f_i}
    x = np.random.default_rng(3).standard_normal((2, 128))
    pos, theta = 70000, 500000.0
    f = theta ** (-np.arange(64) * 2.0 / 128)
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * pos * f)
    np.testing.assert_allclose(step.rope(x, pos, theta), np.concatenate([z.real, z.imag], 1),
                               rtol=1e-12, atol=1e-12)


def test_bf16_rounding_matches_torch_on_float32():
    r = np.random.default_rng(4)
    x = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000),
                        [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2.0 ** -130,
                         3.0e38, 0.0]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = step.round_to_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)
    # ties to even by hand: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert got[20000] == 1.0 and got[20001] == 1 + 2.0 ** -6


def _layer(r, d=32, h_q=4, h_kv=2, d_h=8, f=48, n=30, cap=40, with_sel=True, k_keep=None):
    w = lambda *s: r.standard_normal(s) * 0.2
    k = np.zeros((h_kv, cap, d_h))
    v = np.zeros((h_kv, cap, d_h))
    k[:, :n] = r.standard_normal((h_kv, n, d_h))
    v[:, :n] = r.standard_normal((h_kv, n, d_h))
    kw = {}
    if with_sel:
        idx = np.tile(np.arange(n), (h_kv, 1)) if k_keep is None else k_keep
        ks = np.zeros_like(k)
        vs = np.zeros_like(v)
        ks[:, :idx.shape[1]] = selection.gather(k, idx)
        vs[:, :idx.shape[1]] = selection.gather(v, idx)
        kw = dict(k_sel=ks, v_sel=vs, n_sel=idx.shape[1])
    return step.Layer(np.ones(d), w((h_q + 2 * h_kv) * d_h, d), w(d, h_q * d_h), np.ones(d),
                      w(f, d), w(f, d), w(f, d), 0.1, k, v, n, **kw)


DIMS = dict(n_q_heads=4, n_kv_heads=2, head_dim=8, kv_dtype="f32", eps=1e-5, theta=1e4)


def test_keep_ratio_one_and_dense_mlp_is_bitwise_dense():
    r = np.random.default_rng(5)
    la = _layer(r)
    lb = step.Layer(**{k: getattr(la, k) for k in
                       ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down_t",
                        "threshold", "k_full", "v_full", "n", "k_sel", "v_sel", "n_sel")})
    h = r.standard_normal(32)
    h1 = step.decode_step([la], h, 30, kv_sparse=False, mlp_sparse=False, **DIMS)
    h2 = step.decode_step([lb], h, 30, kv_sparse=True, mlp_sparse=True,
                          masks=[np.ones(48, bool)], **DIMS)
    assert np.array_equal(h1, h2)
    # both buffers received the new row
    assert np.array_equal(lb.k_sel[:, 30], lb.k_full[:, 30]) and lb.n_sel == 31 and lb.n == 31


def test_layer_matches_torch_reference():
    # the same layer built from torch library routines (rms_norm, linear, sdpa,
    # complex RoPE, silu) in float64
    r = np.random.default_rng(6)
    la = _layer(r, with_sel=False)
    h = r.standard_normal(32)
    k0, v0 = la.k_full.copy(), la.v_full.copy()
    got = step.decode_step([la], h, 30, kv_sparse=False, mlp_sparse=False, **DIMS)
    F = torch.nn.functional
    t = torch.from_numpy
    x = F.rms_norm(t(h), (32,), t(la.attn_norm), 1e-5)
    qkv = F.linear(x, t(la.w_qkv))
    q, k, v = qkv[:32].view(4, 8), qkv[32:48].view(2, 8), qkv[48:].view(2, 8)
    f = 1e4 ** (-torch.arange(4, dtype=torch.float64) * 2 / 8)
    rot = torch.polar(torch.ones(4, dtype=torch.float64), 30 * f)

    def rope(z):
        c = torch.complex(z[:, :4], z[:, 4:]) * rot
        return torch.cat([c.real, c.imag], 1)

    q, k = rope(q), rope(k)
    K = torch.cat([t(k0[:, :30]), k[:, None].float().double()], 1)
    V = torch.cat([t(v0[:, :30]), v[:, None].float().double()], 1)
    o = F.scaled_dot_product_attention(q[:, None], K.repeat_interleave(2, 0),
                                       V.repeat_interleave(2, 0))[:, 0]
    hh = t(h) + F.linear(o.reshape(-1), t(la.w_o))
    x2 = F.rms_norm(hh, (32,), t(la.mlp_norm), 1e-5)
    y = F.linear(F.silu(F.linear(x2, t(la.w_gate))) * F.linear(x2, t(la.w_up)), t(la.w_down_t).T)
    np.testing.assert_allclose(got, (hh + y).numpy(), rtol=1e-6, atol=1e-7)


def test_sparse_kv_reads_only_gathered_rows():
    r = np.random.default_rng(7)
    idx = np.array([[0, 1, 5, 9, 28, 29], [0, 1, 2, 17, 28, 29]])
    la = _layer(r, k_keep=idx)
    h = r.standard_normal(32)
    tr = []
    step.decode_step([la], h, 30, kv_sparse=True, mlp_sparse=False, trace=tr, **DIMS)
    from oracle import attention
    q = tr[0]["q"]
    want_k = np.stack([la.k_full[kv, idx[kv]] for kv in range(2)])
    assert np.array_equal(la.k_sel[:, :6], want_k)
    o, _ = attention.attend(q, la.k_sel, la.v_sel, 7, 1 / np.sqrt(8))
    np.testing.assert_array_equal(tr[0]["attn"], o)
    # and differs from attending over the full cache
    o_full, _ = attention.attend(q, la.k_full, la.v_full, 31, 1 / np.sqrt(8))
    assert np.abs(o_full - o).max() > 1e-3


def test_ragged_layer_appends_per_head_and_equals_uniform_when_equal():
    r = np.random.default_rng(8)
    la = _layer(r)
    lb = step.Layer(**{k: copy.deepcopy(getattr(la, k)) for k in
                       ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down_t",
                        "threshold", "k_full", "v_full", "n", "k_sel", "v_sel", "n_sel")},
                    n_sel_heads=[la.n_sel, la.n_sel])
    h = r.standard_normal(32)
    ha = step.decode_step([la], h, 30, kv_sparse=True, mlp_sparse=False, **DIMS)
    hb = step.decode_step([lb], h, 30, kv_sparse=True, mlp_sparse=False, **DIMS)
    assert np.array_equal(ha, hb) and lb.n_sel_heads == [31, 31]
    # unequal lengths: head 0 keeps 10 rows, head 1 all 30; each appends at its own row
    lc = _layer(np.random.default_rng(8))
    lc.n_sel_heads = [10, 30]
    tr = []
    step.decode_step([lc], h, 30, kv_sparse=True, mlp_sparse=False, trace=tr, **DIMS)
    assert lc.n_sel_heads == [11, 31]
    assert np.array_equal(lc.k_sel[0, 10], lc.k_full[0, 30])
    assert np.array_equal(lc.k_sel[1, 30], lc.k_full[1, 30])
    from oracle import attention
    o, _ = attention.attend_ragged(tr[0]["q"], lc.k_sel, lc.v_sel, [11, 31], 1 / np.sqrt(8))
    assert np.array_equal(tr[0]["attn"], o)
