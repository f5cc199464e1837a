"""Pins of the TEAL oracle: threshold-based activation sparsity on every
projection's input ("Where Activation Sparsity and KV-Cache Sparsity Cross in
LLM Decoding", §3.2 "Sparse Branches" and §4.1 "Setup")."""

import copy

import numpy as np

from oracle import cats, step, teal
from test_oracle_step import DIMS, _layer


def test_negative_threshold_is_the_dense_projection_bitwise():
    r = np.random.default_rng(11)
    w = r.standard_normal((24, 40))
    x = r.standard_normal(40)
    y, mask, idx = teal.teal_linear(w, x, -1.0)
    assert mask.all() and len(idx) == 40
    assert np.array_equal(y, w @ x)


def test_closed_form_two_channels():
    w = np.array([[1.0, 2.0], [3.0, 4.0]])
    y, mask, idx = teal.teal_linear(w, np.array([0.5, -2.0]), 1.0)
    assert mask.tolist() == [False, True] and idx.tolist() == [1]
    assert y.tolist() == [-4.0, -8.0]


def test_threshold_is_strict_and_decided_in_float32():
    x = np.array([0.25, -0.25, 0.2500001, 0.3, -0.1])
    m = teal.teal_mask(x.astype(np.float32), 0.25)
    # |x| == t is dropped; 0.2500001 rounds to a float32 above 0.25 and is kept
    assert m.tolist() == [False, False, True, True, False]


def test_all_dropped_gives_zero():
    r = np.random.default_rng(12)
    w = r.standard_normal((8, 16))
    y, mask, idx = teal.teal_linear(w, r.standard_normal(16) * 0.1, 100.0)
    assert not mask.any() and len(idx) == 0 and np.array_equal(y, np.zeros(8))


def test_gathered_columns_equal_masked_dense():
    r = np.random.default_rng(13)
    w = r.standard_normal((30, 64))
    x = r.standard_normal(64)
    y, mask, idx = teal.teal_linear(w, x, 0.7)
    assert 10 < len(idx) < 54
    np.testing.assert_allclose(teal.linear_gathered_loops(w.T, x, idx), y, rtol=1e-12, atol=1e-12)


def test_layer_with_negative_thresholds_is_the_dense_layer_bitwise():
    r = np.random.default_rng(14)
    la = _layer(r, with_sel=False)
    lb = copy.deepcopy(la)
    h = r.standard_normal(32)
    want = step.decode_step([la], h, 30, kv_sparse=False, mlp_sparse=False, **DIMS)
    got = teal.teal_step([lb], h, 30, [(-1.0, -1.0, -1.0, -1.0)], kv_sparse=False, **DIMS)
    assert np.array_equal(got, want)
    assert np.array_equal(la.k_full, lb.k_full) and lb.n == la.n


def _inputs(layer, states, pos):
    """The four projection inputs of the layer for each state (dense pass)."""
    tr = []
    for h in states:
        teal.teal_layer(copy.deepcopy(layer), h, pos, (-1.0,) * 4, kv_sparse=False, trace=tr,
                        **DIMS)
    return [np.concatenate([t[k].ravel() for t in tr]) for k in ("x", "attn", "x2", "hmid")]


def test_calibrated_thresholds_keep_the_target_fraction_of_every_input():
    # thresholds calibrated for 50% keep on one set of states keep about half of
    # each of the four inputs on fresh states (the pages' TEAL setting: 50% keep
    # in all seven projections)
    r = np.random.default_rng(15)
    la = _layer(r, with_sel=False)
    cal = [r.standard_normal(32) for _ in range(64)]
    ts = [cats.calibrate_threshold(np.abs(v).astype(np.float32), 0.5) for v in _inputs(la, cal, 30)]
    # exact on the calibration set itself (tie-free data)
    for v, t in zip(_inputs(la, cal, 30), ts):
        assert (np.abs(v.astype(np.float32)) > np.float32(t)).sum() == v.size - round(0.5 * v.size)
    fresh = [r.standard_normal(32) for _ in range(64)]
    tr = []
    for h in fresh:
        teal.teal_layer(copy.deepcopy(la), h, 30, ts, kv_sparse=False, trace=tr, **DIMS)
    for k in range(4):
        frac = np.mean([t["masks"][k].mean() for t in tr])
        assert 0.4 < frac < 0.6, (k, frac)


def test_injected_masks_replace_the_decisions():
    r = np.random.default_rng(16)
    la = _layer(r, with_sel=False)
    h = r.standard_normal(32)
    masks = [np.zeros(32, bool), np.zeros(32, bool), np.zeros(32, bool), np.zeros(48, bool)]
    got = teal.teal_layer(copy.deepcopy(la), h, 30, (-1.0,) * 4, kv_sparse=False, masks=masks,
                          **DIMS)
    # every projection reads nothing: q = k = v = 0, o = mean of V with the new
    # zero row, h unchanged by O and the MLP
    assert np.array_equal(got, h)


def test_each_mask_acts_on_its_own_projection():
    # attention input dropped entirely: q = k = v = 0, so the softmax over the
    # n + 1 rows is uniform and o is the plain mean of V (the appended row is
    # zero); O keeps all of o; the MLP input is dropped, so gate = up = 0 and
    # the down input SiLU(0) * 0 is zero: h' = h + W_o mean(V)
    r = np.random.default_rng(17)
    la = _layer(r, with_sel=False)
    h = r.standard_normal(32)
    v0 = la.v_full[:, :30].copy()
    masks = [np.zeros(32, bool), np.ones(32, bool), np.zeros(32, bool), np.ones(48, bool)]
    got = teal.teal_layer(la, h, 30, (-1.0,) * 4, kv_sparse=False, masks=masks, **DIMS)
    mean_v = v0.sum(axis=1) / 31.0                      # [h_kv, d_h]
    o = np.repeat(mean_v, 2, axis=0).reshape(-1)        # G = 2 query heads per KV head
    np.testing.assert_allclose(got, h + la.w_o @ o, rtol=1e-12, atol=1e-12)
    assert not la.k_full[:, 30].any() and not la.v_full[:, 30].any()
    # and the converse: attention input and O input kept but O's mask empty
    lb = _layer(np.random.default_rng(17), with_sel=False)
    masks = [np.ones(32, bool), np.zeros(32, bool), np.ones(32, bool), np.zeros(48, bool)]
    got = teal.teal_layer(lb, h, 30, (-1.0,) * 4, kv_sparse=False, masks=masks, **DIMS)
    assert np.array_equal(got, h)
