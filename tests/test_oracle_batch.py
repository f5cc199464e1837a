"""Pins of the batch oracle: B sequences sharing weights, union channel masks
("Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding",
§3.3 "Dispatch and batching", §4.4 "Batching")."""

import copy

import numpy as np

from oracle import batch, step
from test_oracle_step import DIMS, _layer


def _seq_layers(r, batch_size, n_layers=2):
    """Layers whose weights are shared and whose caches differ per sequence."""
    base = [_layer(r) for _ in range(n_layers)]
    out = []
    for b in range(batch_size):
        seq = []
        for L in base:
            c = copy.copy(L)  # shares the weight arrays
            c.k_full = r.standard_normal(L.k_full.shape)
            c.v_full = r.standard_normal(L.v_full.shape)
            c.k_sel = c.k_full.copy()
            c.v_sel = c.v_full.copy()
            c.n, c.n_sel = 30 - b, 30 - b
            seq.append(c)
        out.append(seq)
    return out


def test_batch_of_one_is_the_single_step_bitwise():
    r = np.random.default_rng(40)
    seq = _seq_layers(r, 1)
    ref = copy.deepcopy(seq[0])
    h = r.standard_normal(32)
    got, unions = batch.decode_step_batch(seq, [h], [30], kv_sparse=True, mlp_sparse=True, **DIMS)
    tr = []
    want = step.decode_step(ref, h, 30, kv_sparse=True, mlp_sparse=True, trace=tr, **DIMS)
    assert np.array_equal(got[0], want)
    for li in range(2):
        assert np.array_equal(unions[li], tr[li]["mask"])


def test_sequences_are_independent():
    # changing sequence 1's cache and state leaves sequence 0's result as is
    r = np.random.default_rng(41)
    seq = _seq_layers(r, 3)
    hs = r.standard_normal((3, 32))
    a, _ = batch.decode_step_batch(copy.deepcopy(seq), hs, [30, 29, 28], kv_sparse=False,
                                   mlp_sparse=True, **DIMS)
    seq2 = copy.deepcopy(seq)
    for L in seq2[1]:
        L.k_full[:] = r.standard_normal(L.k_full.shape)
    hs2 = hs.copy()
    hs2[1] = r.standard_normal(32)
    b, _ = batch.decode_step_batch(seq2, hs2, [30, 29, 28], kv_sparse=False, mlp_sparse=True,
                                   **DIMS)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    assert not np.array_equal(a[1], b[1])


def test_union_closed_forms():
    m = np.array([1, 0, 1, 0, 0, 1], bool)
    assert np.array_equal(batch.union_mask([m, m, m]), m)
    d = [np.eye(6, dtype=bool)[i] for i in range(6)]     # disjoint one-hot masks
    assert batch.union_mask(d).all() and batch.union_fraction(d[:3]) == 0.5
    assert batch.union_fraction([np.zeros(8, bool)] * 4) == 0.0


def test_union_of_independent_masks_matches_closed_form():
    # keep probability 0.5 per channel and sequence: E[u_B] = 1 - 0.5^B
    r = np.random.default_rng(42)
    n = 400000
    # (and keep 0.3: 1 - 0.7^B, which tells keep from drop probabilities apart)
    for keep, B, want in ((0.5, 1, 0.5), (0.5, 4, 0.9375), (0.5, 8, 1 - 0.5 ** 8),
                          (0.3, 4, 1 - 0.7 ** 4), (0.3, 2, 0.51)):
        got = batch.union_fraction(r.random((B, n)) < keep)
        assert abs(batch.independent_union_fraction(keep, B) - want) < 1e-12
        sigma = np.sqrt(want * (1 - want) / n)
        assert abs(got - want) < 5 * sigma + 1e-12, (keep, B, got, want)


def test_union_fraction_of_real_step_masks_is_bounded():
    # u_B lies between the largest single keep fraction and min(1, sum of them)
    r = np.random.default_rng(43)
    seq = _seq_layers(r, 4, n_layers=1)
    hs = r.standard_normal((4, 32))
    tr = []
    _, unions = batch.decode_step_batch(seq, hs, [30, 29, 28, 27], kv_sparse=False,
                                        mlp_sparse=True, trace=tr, **DIMS)
    fr = [t[0]["mask"].mean() for t in tr]
    u = unions[0].mean()
    assert max(fr) <= u <= min(1.0, sum(fr))


def test_each_sequence_is_its_own_single_step():
    # distinct positions, caches and states: sequence b equals the single-step
    # oracle run on sequence b alone
    r = np.random.default_rng(44)
    seq = _seq_layers(r, 3)
    ref = copy.deepcopy(seq)
    hs = r.standard_normal((3, 32))
    pos = [30, 29, 28]
    got, _ = batch.decode_step_batch(seq, hs, pos, kv_sparse=True, mlp_sparse=False, **DIMS)
    for b in range(3):
        want = step.decode_step(ref[b], hs[b], pos[b], kv_sparse=True, mlp_sparse=False, **DIMS)
        assert np.array_equal(got[b], want), b
