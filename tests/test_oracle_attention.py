"""Pins of the oracle's decode attention and split-K combine."""

import numpy as np
import torch

from oracle import attention as att


def _rand(seed, h_q=4, h_kv=2, n=17, d_h=8):
    r = np.random.default_rng(seed)
    return (r.standard_normal((h_q, d_h)), r.standard_normal((h_kv, n + 2, d_h)),
            r.standard_normal((h_kv, n + 2, d_h)))


def test_matches_python_loops():
    q, k, v = _rand(1)
    o, l = att.attend(q, k, v, 17, 0.3)
    o2, l2 = att.attend_loops(q, k, v, 17, 0.3)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l, l2, rtol=1e-12)


def test_matches_torch_sdpa_gqa():
    # library routine: torch scaled_dot_product_attention, float64, K/V repeated per group
    q, k, v = _rand(2, h_q=8, h_kv=2, n=33, d_h=16)
    o, _ = att.attend(q, k, v, 33, 0.25)
    kt = torch.from_numpy(k[:, :33]).repeat_interleave(4, dim=0)
    vt = torch.from_numpy(v[:, :33]).repeat_interleave(4, dim=0)
    qt = torch.from_numpy(q)[:, None, :]
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.25)[:, 0]
    np.testing.assert_allclose(o, want.numpy(), rtol=1e-12, atol=1e-14)


def test_special_cases():
    q, k, v = _rand(3)
    vc = np.full_like(v, 2.5)
    o, _ = att.attend(q, k, vc, 17, 0.3)
    np.testing.assert_allclose(o, 2.5, rtol=1e-14)              # constant V
    o, l = att.attend(q, k, v, 1, 0.3)                           # one row
    np.testing.assert_allclose(o, v[[0, 0, 1, 1], 0], rtol=1e-14)
    np.testing.assert_allclose(l, (k[[0, 0, 1, 1], 0] * q).sum(1) * 0.3, rtol=1e-13)
    o, l = att.attend(np.zeros_like(q), k, v, 17, 0.3)            # q = 0: mean of V
    np.testing.assert_allclose(o, v[[0, 0, 1, 1], :17].mean(1), rtol=1e-13)
    np.testing.assert_allclose(l, np.log(17.0))


def test_two_key_closed_form():
    # logits 0 and ln 3: weights 1/4 and 3/4
    q = np.array([[1.0, 0.0]])
    k = np.array([[[0.0, 0.0], [np.log(3.0) / 0.5, 0.0]]])
    v = np.array([[[4.0, 0.0], [0.0, 8.0]]])
    o, l = att.attend(q, k, v, 2, 0.5)
    np.testing.assert_allclose(o, [[1.0, 6.0]], rtol=1e-14)
    np.testing.assert_allclose(l, [np.log(4.0)], rtol=1e-14)


def test_combine_of_any_partition_equals_unsplit():
    q, k, v = _rand(4, n=101)
    o, l = att.attend(q, k, v, 101, 0.2)
    r = np.random.default_rng(0)
    for _ in range(5):
        cuts = np.sort(r.integers(0, 102, size=7))
        bounds = np.concatenate([[0], cuts, [101]])  # includes empty chunks
        m, ll, acc = att.partials(q, k, v, bounds, 0.2)
        o2, l2 = att.combine(m, ll, acc)
        np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l2, l, rtol=1e-12)


def test_combine_two_chunks_by_hand():
    # chunk A: m=0, l=1, acc=[1]; chunk B: m=ln 2, l=1, acc=[3] -> weights 1, 2
    m = np.array([[0.0, np.log(2.0)]])
    l = np.ones((1, 2))
    acc = np.array([[[1.0], [3.0]]])
    o, lse = att.combine(m, l, acc)
    np.testing.assert_allclose(o, [[(1 + 6) / 3]])
    np.testing.assert_allclose(lse, [np.log(3.0)])


def test_ragged_lengths_match_per_head_loops():
    r = np.random.default_rng(31)
    q = r.standard_normal((6, 16))
    k = r.standard_normal((3, 40, 16))
    v = r.standard_normal((3, 40, 16))
    lens = [7, 40, 1]
    out, lse = att.attend_ragged(q, k, v, lens, 0.25)
    for kv, n in enumerate(lens):
        o, l = att.attend_loops(q[2 * kv:2 * kv + 2], k[kv:kv + 1], v[kv:kv + 1], n, 0.25)
        np.testing.assert_allclose(out[2 * kv:2 * kv + 2], o, rtol=1e-12, atol=1e-12)
    # one row: the output is that row of V
    np.testing.assert_allclose(out[4:6], np.tile(v[2, 0], (2, 1)), rtol=1e-12)
    # equal lengths: the uniform attention, bit for bit
    o2, _ = att.attend_ragged(q, k, v, [40, 40, 40], 0.25)
    assert np.array_equal(o2, att.attend(q, k, v, 40, 0.25)[0])
