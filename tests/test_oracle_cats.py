"""Pins of the oracle's CATS sparse MLP (SiLU gate, |a| > t mask, masked-dense
SwiGLU) and its percentile threshold calibration, following "Sensitivity-Aware
Thresholding and Token Routing for Activation Sparsification in Large
Language Models" (CATS runtime masking, text around Eq. 6)."""

import numpy as np
import pytest
import torch

from oracle import cats


def _mlp(seed, d=24, f=40):
    r = np.random.default_rng(seed)
    return (r.standard_normal(d), r.standard_normal((f, d)) * 0.3,
            r.standard_normal((f, d)) * 0.3, r.standard_normal((f, d)) * 0.3)


def test_silu_special_points():
    g = np.array([0.0, np.log(3.0), -np.log(3.0), 40.0, -40.0])
    a = cats.silu(g)
    assert a[0] == 0.0
    np.testing.assert_allclose(a[1], 0.75 * np.log(3.0), rtol=1e-15)   # sigmoid(ln 3) = 3/4
    np.testing.assert_allclose(a[2], -0.25 * np.log(3.0), rtol=1e-15)
    np.testing.assert_allclose(a[3], 40.0, rtol=1e-15)
    assert abs(a[4]) < 1e-15


def test_dense_matches_torch_swiglu():
    x, wg, wu, wd = _mlp(1)
    y, a, mask, idx = cats.cats_mlp(x, wg, wu, wd, -1.0)
    t = lambda z: torch.from_numpy(np.asarray(z))
    F = torch.nn.functional
    want = F.linear(F.silu(F.linear(t(x), t(wg))) * F.linear(t(x), t(wu)), t(wd).T)
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=1e-14)
    assert mask.all() and idx.tolist() == list(range(40))


@pytest.mark.parametrize("t", [-1.0, -0.0, 0.0])
def test_threshold_nonpositive_is_bitwise_dense(t):
    x, wg, wu, wd = _mlp(2)
    y, *_ = cats.cats_mlp(x, wg, wu, wd, t)
    assert np.array_equal(y, cats.dense_swiglu(x, wg, wu, wd))


def test_gathered_equals_masked_dense():
    x, wg, wu, wd = _mlp(3)
    for t in (0.05, 0.2, 0.5):
        y, a, mask, idx = cats.cats_mlp(x, wg, wu, wd, t)
        assert 0 < idx.size < 40
        np.testing.assert_allclose(y, cats.mlp_gathered_loops(x, wg, wu, wd, idx),
                                   rtol=1e-12, atol=1e-13)


def test_mask_is_strict_and_float32():
    a = np.array([0.5, -0.5, 0.49999997, -0.7, 0.0], np.float32)
    m = cats.cats_mask(a, 0.5)
    assert m.tolist() == [False, False, False, True, False]
    with pytest.raises(TypeError):
        cats.cats_mask(a.astype(np.float64), 0.5)


def test_kept_indices_ascending():
    m = np.array([0, 1, 1, 0, 1], bool)
    assert cats.kept_indices(m).tolist() == [1, 2, 4]


@pytest.mark.parametrize("s", [0.0, 0.3, 0.5, 0.7, 1.0])
def test_calibration_realizes_exact_sparsity(s):
    v = np.random.default_rng(4).permutation(np.arange(1, 1001, dtype=np.float32) * 1e-3)
    t = cats.calibrate_threshold(v, s)
    k = int(round(s * 1000))
    if k == 0:
        assert t < 0
    else:
        assert int((v <= np.float32(t)).sum()) == k
        # the mask keeps exactly the rest
        assert int(cats.cats_mask(v, t).sum()) == 1000 - k
