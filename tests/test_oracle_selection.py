"""Pins of the oracle's KV selection (one-time observation-window scoring,
per-KV-head top-k and gather), following "Where Activation Sparsity and
KV-Cache Sparsity Cross in LLM Decoding", §4.1."""

import numpy as np
import pytest
import torch

import synth
from oracle import selection as sel


def _tiny(seed, h_q=4, h_kv=2, n=40, w=6, d_h=8):
    r = np.random.default_rng(seed)
    q = r.standard_normal((h_q, w, d_h))
    k = r.standard_normal((h_kv, n + 3, d_h))
    return q, k


def test_scores_match_python_loops():
    q, k = _tiny(1)
    n = 40
    s = sel.window_scores(q, k, n, 1 / np.sqrt(8))
    s_loop = sel.window_scores_loops(q, k, n, 1 / np.sqrt(8))
    np.testing.assert_allclose(s, s_loop, rtol=1e-12, atol=1e-14)


def test_scores_match_torch_causal_softmax():
    # a library routine: torch's softmax over the masked logit matrix, float64
    q, k = _tiny(2, h_q=6, h_kv=3, n=50, w=9, d_h=16)
    n, w, g = 50, 9, 2
    s = sel.window_scores(q, k, n, 0.25)
    want = torch.zeros(3, n, dtype=torch.float64)
    qt, kt = torch.from_numpy(q), torch.from_numpy(k)
    rows = torch.arange(w)[:, None] + (n - w)
    cols = torch.arange(n)[None, :]
    for h in range(6):
        z = (qt[h] @ kt[h // g, :n].T) * 0.25
        z = z.masked_fill(cols > rows, float("-inf"))
        want[h // g] += torch.softmax(z, dim=-1).sum(0)
    np.testing.assert_allclose(s, want.numpy(), rtol=1e-12, atol=1e-15)


def test_scores_sum_to_group_times_window():
    q, k = _tiny(3, h_q=8, h_kv=2, n=300, w=32, d_h=16)
    s = sel.window_scores(q, k, 300, 0.25)
    np.testing.assert_allclose(s.sum(axis=1), 4 * 32, rtol=1e-12)


def test_zero_keys_give_harmonic_closed_form():
    # all logits equal: query at position p spreads 1/(p+1) over keys 0..p
    h_q, h_kv, n, w, d_h = 4, 2, 20, 5, 8
    q = np.random.default_rng(4).standard_normal((h_q, w, d_h))
    k = np.zeros((h_kv, n, d_h))
    s = sel.window_scores(q, k, n, 1.0)
    pos = n - w + np.arange(w)
    want = np.array([sum(1.0 / (p + 1) for p in pos if p >= j) for j in range(n)]) * 2
    np.testing.assert_allclose(s, np.tile(want, (h_kv, 1)), rtol=1e-13)


def test_scale_and_group_mapping_closed_form():
    # one window query per head; only head 2 (group 1 -> KV head 1) is nonzero and
    # its logit on key 1 exceeds the others by ln 3: weights 3/(n+2) vs 1/(n+2)
    h_q, h_kv, n, d_h = 4, 2, 6, 4
    q = np.zeros((h_q, 1, d_h))
    k = np.zeros((h_kv, n, d_h))
    q[2, 0, 0] = 1.0
    k[1, 1, 0] = np.log(3.0) * np.sqrt(d_h)
    s = sel.window_scores(q, k, n, 1 / np.sqrt(d_h))
    np.testing.assert_allclose(s[0], 2.0 / n)                      # heads 0, 1: uniform
    want1 = np.full(n, 1.0 / n + 1.0 / (n + 2))                    # head 3 uniform + head 2
    want1[1] = 1.0 / n + 3.0 / (n + 2)
    np.testing.assert_allclose(s[1], want1, rtol=1e-13)


def test_lse_definition_special_case():
    # keys all zero: lse of the query at position p is log(p + 1)
    q = np.ones((2, 3, 4))
    k = np.zeros((1, 10, 4))
    lse = sel.window_lse(q, k, 10, 1.0)
    np.testing.assert_allclose(lse, np.log(np.array([8.0, 9.0, 10.0]))[None].repeat(2, 0))


def test_topk_matches_loops_with_ties():
    r = np.random.default_rng(5)
    s = r.integers(0, 6, size=(3, 60)).astype(np.float32)  # many ties
    for k_keep in (10, 20, 37, 59):
        a = sel.select_indices(s, 60, 5, 4, k_keep)
        b = sel.select_indices_loops(s, 60, 5, 4, k_keep)
        np.testing.assert_array_equal(a, b)


def test_topk_forced_entries_and_order():
    r = np.random.default_rng(6)
    s = r.random((2, 100)).astype(np.float32)
    s[:, :4] = 0.0          # sinks with the lowest scores must still be kept
    s[:, -8:] = 0.0         # so must the window
    idx = sel.select_indices(s, 100, 8, 4, 30)
    for kv, row in enumerate(idx):
        assert np.all(np.diff(row) > 0)
        assert set(range(4)) <= set(row) and set(range(92, 100)) <= set(row)
        chosen = set(row) - set(range(4)) - set(range(92, 100))
        assert len(chosen) == 18
        # the chosen ones are exactly the 18 best candidates (no ties in random data)
        best = 4 + np.argsort(-s[kv, 4:92].astype(np.float64))[:18]
        assert chosen == set(best.tolist())


def test_all_equal_scores_pick_lowest_positions():
    s = np.full((2, 50), 0.5, np.float32)
    idx = sel.select_indices(s, 50, 6, 4, 20)
    want = list(range(4)) + list(range(4, 14)) + list(range(44, 50))
    assert idx.tolist() == [want, want]


def test_keep_ratio_one_is_identity():
    q, k = _tiny(7)
    v = k + 1
    s, idx, ks, vs = sel.select_kv(q, k, v, 40, 4, 40)
    assert idx.tolist() == [list(range(40))] * 2
    np.testing.assert_array_equal(ks, k[:, :40])
    np.testing.assert_array_equal(vs, v[:, :40])


def test_bad_budget_rejected():
    s = np.zeros((1, 50), np.float32)
    with pytest.raises(ValueError):
        sel.select_indices(s, 50, 8, 4, 11)


def test_planted_keys_recovered():
    # retrieval stand-in: keys planted along the window queries' mean direction
    # must all survive a 16% selection in every KV head
    wl = synth.L8B_KV_32K
    import dataclasses
    small = dataclasses.replace(wl, n_q_heads=8, n_kv_heads=2, n_ctx=4096, n_planted=32)
    n = small.n_ctx
    k, v = synth.kv_cache(small, 0, n, n)
    qw = synth.window_queries(small, 0)
    pos = synth.plant_keys(small, 0, k, n, qw)
    s, idx, _, _ = sel.select_kv(qw, k, v, n, small.n_sink, small.k_keep)
    for kv in range(small.n_kv_heads):
        assert set(pos.tolist()) <= set(idx[kv].tolist())


def test_window_indices_definition():
    # brute force: the first n_sink rows and the last n_keep - n_sink rows
    for n, s_, k in [(100, 4, 30), (100, 0, 30), (10, 4, 4), (7, 4, 10), (50, 4, 50)]:
        got = sel.window_indices(n, s_, k).tolist()
        if k >= n:
            want = list(range(n))
        else:
            want = sorted(set(range(s_)) | set(range(n - (k - s_), n)))
        assert got == want
        assert len(got) == min(k, n)


def test_window_attention_equals_attention_over_its_rows():
    # the window reads its rows in place; attending over them equals attending
    # over a gathered copy of them
    from oracle import attention
    r = np.random.default_rng(9)
    q = r.standard_normal((4, 8))
    k = r.standard_normal((2, 60, 8))
    v = r.standard_normal((2, 60, 8))
    idx = sel.window_indices(60, 4, 20)
    o1, l1 = attention.attend(q, k[:, idx], v[:, idx], len(idx), 0.3)
    z = np.einsum("hd,hjd->hj", q, np.repeat(k[:, idx], 2, axis=0)) * 0.3
    w = np.exp(z - z.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    np.testing.assert_allclose(o1, np.einsum("hj,hjd->hd", w, np.repeat(v[:, idx], 2, axis=0)),
                               rtol=1e-12)


def test_ragged_budgets_equal_to_one_k_are_the_uniform_selection():
    r = np.random.default_rng(21)
    s = r.random((4, 300)).astype(np.float32)
    want = sel.select_indices(s, 300, 16, 4, 90)
    got = sel.select_indices_ragged(s, 300, 16, 4, [90] * 4)
    assert all(np.array_equal(g, w) for g, w in zip(got, want))


def test_ragged_budgets_per_head():
    r = np.random.default_rng(22)
    s = r.random((3, 200)).astype(np.float32)
    got = sel.select_indices_ragged(s, 200, 8, 2, [10, 500, 64])
    assert [len(g) for g in got] == [10, 200, 64]
    assert np.array_equal(got[1], np.arange(200))  # k >= n keeps every row
    for kv, k in ((0, 10), (2, 64)):
        assert np.array_equal(got[kv], sel.select_indices(s[kv:kv + 1], 200, 8, 2, k)[0])
        # sinks and window are forced, the rest are the top scores of the candidates
        assert set(range(2)) <= set(got[kv]) and set(range(192, 200)) <= set(got[kv])


def test_catekv_budgets_closed_form():
    # the page's benchmark setting: adaptive heads keep everything (eta = 1),
    # consistent heads a 2048-entry budget; with 3 of 8 KV heads adaptive at
    # 128K the kept fraction is (3 n + 5 * 2048) / (8 n)
    n = 131072
    ks = sel.catekv_budgets(n, [1, 0, 0, 1, 0, 0, 1, 0], 2048, 1.0)
    assert ks == [n, 2048, 2048, n, 2048, 2048, n, 2048]
    assert abs(sum(ks) / (8 * n) - (3 * n + 5 * 2048) / (8 * n)) < 1e-15
    assert sel.catekv_budgets(1000, [1, 0], 2048, 0.5) == [500, 1000]


def test_gather_ragged_hand_built_rows():
    # row j of head kv holds the value 1000 kv + j in every channel, so each
    # gathered row names the head and position it came from
    h_kv, cap, d_h = 3, 9, 4
    cache = (1000.0 * np.arange(h_kv)[:, None, None] + np.arange(cap)[None, :, None]
             + np.zeros((1, 1, d_h)))
    idx = [np.array([0, 3]), np.array([1]), np.array([0, 2, 4, 8])]
    got = sel.gather_ragged(cache, idx)
    want = [[0, 3], [1001], [2000, 2002, 2004, 2008]]
    assert [g.shape for g in got] == [(2, d_h), (1, d_h), (4, d_h)]
    for g, w in zip(got, want):
        assert np.array_equal(g, np.repeat(np.array(w, float)[:, None], d_h, axis=1))


def test_gather_ragged_equal_budgets_is_the_uniform_gather():
    r = np.random.default_rng(23)
    n, h_kv, d_h = 200, 4, 8
    s = r.random((h_kv, n)).astype(np.float32)
    cache = r.standard_normal((h_kv, n + 5, d_h))
    idx_u = sel.select_indices(s, n, 8, 2, 50)
    idx_r = sel.select_indices_ragged(s, n, 8, 2, [50] * h_kv)
    want = sel.gather(cache, idx_u)
    got = sel.gather_ragged(cache, idx_r)
    for kv in range(h_kv):
        assert np.array_equal(got[kv], want[kv])


def test_gather_ragged_matches_a_per_head_loop():
    r = np.random.default_rng(24)
    n, h_kv, d_h = 120, 5, 4
    s = r.random((h_kv, n)).astype(np.float32)
    cache = r.standard_normal((h_kv, n, d_h))
    budgets = [12, 120, 40, 13, 77]
    idx = sel.select_indices_ragged(s, n, 6, 3, budgets)
    got = sel.gather_ragged(cache, idx)
    for kv in range(h_kv):
        assert len(got[kv]) == min(budgets[kv], n)
        for r_, j in enumerate(idx[kv]):
            for c in range(d_h):
                assert got[kv][r_, c] == cache[kv, j, c]
