"""GPU parity of sd_select_kv: window scores against the float64 oracle, the
per-KV-head top-k bit-exact on the oracle's float32 scores (SD_SCORES_IN),
the gather bit-exact, planted-key recall, and the degenerate cases."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import selection as osel

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import DEV, TOL, dims_for, rel_l2, to_dev, to_host, workspace  # noqa: E402


class Sel:
    """Device buffers for one selection call."""

    def __init__(self, wl, k, v, n, cap, k_keep, cap_sel=None):
        self.wl, self.n, self.cap, self.k_keep = wl, n, cap, k_keep
        self.k_eff = min(k_keep, n)
        self.cap_sel = cap_sel or self.k_eff + 4
        self.dims = dims_for(wl)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.kd, self.vd = to_dev(k, wl.dtype), to_dev(v, wl.dtype)
        self.ks = torch.zeros(wl.n_kv_heads, self.cap_sel, wl.head_dim, dtype=tdt, device=DEV)
        self.vs = torch.zeros_like(self.ks)
        self.scores = torch.empty(wl.n_kv_heads, n, device=DEV)
        self.idx = torch.empty(wl.n_kv_heads, self.k_eff, dtype=torch.int32, device=DEV)
        self.ws = workspace(self.dims, n, max(64, wl.window))

    def run(self, q_win=None, scores_in=None, w=None, n_sink=None):
        wl = self.wl
        w = wl.window if w is None else w
        n_sink = wl.n_sink if n_sink is None else n_sink
        flags = 0
        qd = None
        if scores_in is not None:
            self.scores.copy_(torch.from_numpy(np.ascontiguousarray(scores_in, np.float32)))
            flags = sd.SD_SCORES_IN
        else:
            qd = to_dev(q_win)
        sd.sd_select_kv(self.dims, self.kd, self.vd, self.cap, self.n, qd, w, n_sink, self.k_keep,
                        self.scores, self.idx, self.ks, self.vs, self.cap_sel, flags, self.ws)
        torch.cuda.synchronize()
        return to_host(self.scores), self.idx.cpu().numpy()


def _tiny(n=2048, cap=None, seed_layer=0):
    wl = synth.TINY
    cap = cap or n + 16
    k, v = synth.kv_cache(wl, seed_layer, n, cap)
    return wl, k, v, synth.window_queries(wl, seed_layer), cap


def test_tiny_scores_match_oracle():
    wl, k, v, qw, cap = _tiny()
    s = Sel(wl, k, v, 2048, cap, wl.k_keep)
    got, _ = s.run(qw)
    want = osel.window_scores(qw, k, 2048, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(got, want) <= TOL["f32"]
    # each window query's softmax sums to one: G*w per KV head
    np.testing.assert_allclose(got.sum(1), 2 * wl.window, rtol=1e-5)


@pytest.mark.parametrize("n,w,n_sink,k_keep", [(2048, 32, 4, 512), (2049, 32, 4, 513),
                                               (777, 5, 0, 100), (300, 32, 4, 36),
                                               (1000, 1, 1, 2), (5000, 64, 4, 1500)])
def test_topk_bit_exact_on_oracle_scores(n, w, n_sink, k_keep):
    wl, k, v, _, cap = _tiny(n)
    r = np.random.default_rng(n + k_keep)
    scores = r.random((wl.n_kv_heads, n)).astype(np.float32)
    s = Sel(wl, k, v, n, cap, k_keep)
    _, idx = s.run(scores_in=scores, w=w, n_sink=n_sink)
    assert np.array_equal(idx, osel.select_indices(scores, n, w, n_sink, k_keep))


@pytest.mark.parametrize("levels", [1, 2, 7, 1000])
def test_topk_ties_go_to_lower_position(levels):
    wl, k, v, _, cap = _tiny(3000)
    r = np.random.default_rng(levels)
    scores = (r.integers(0, levels, (wl.n_kv_heads, 3000)) * 0.25).astype(np.float32)
    scores[0, 100:200] = -0.0      # signed zeros tie with +0
    scores[1, 50:60] = -3.5        # negative scores (caller-given) rank lowest
    s = Sel(wl, k, v, 3000, cap, 700)
    _, idx = s.run(scores_in=scores)
    assert np.array_equal(idx, osel.select_indices(scores, 3000, wl.window, wl.n_sink, 700))


# Long contexts use the chunked top-k (chunks of 4096 positions, several
# workgroups per KV head); these cases span chunk boundaries, a ragged last
# chunk, ties across chunks, and the degenerate budgets.
@pytest.mark.parametrize("n,w,n_sink,k_keep", [(9000, 32, 4, 1000), (20000, 32, 4, 3000),
                                               (40961, 64, 0, 4097), (16384, 32, 4, 36),
                                               (12289, 1, 1, 12000), (131072, 32, 4, 13107)])
def test_chunked_topk_bit_exact_on_oracle_scores(n, w, n_sink, k_keep):
    wl, k, v, _, cap = _tiny(n)
    r = np.random.default_rng(n + k_keep)
    scores = r.random((wl.n_kv_heads, n)).astype(np.float32)
    s = Sel(wl, k, v, n, cap, k_keep)
    _, idx = s.run(scores_in=scores, w=w, n_sink=n_sink)
    assert np.array_equal(idx, osel.select_indices(scores, n, w, n_sink, k_keep))


@pytest.mark.parametrize("levels", [1, 2, 7, 1000])
def test_chunked_topk_ties_go_to_lower_position(levels):
    n, k_keep = 20000, 5000
    wl, k, v, _, cap = _tiny(n)
    r = np.random.default_rng(100 + levels)
    scores = (r.integers(0, levels, (wl.n_kv_heads, n)) * 0.25).astype(np.float32)
    scores[0, 4000:4200] = -0.0    # signed zeros across a chunk boundary
    s = Sel(wl, k, v, n, cap, k_keep)
    _, idx = s.run(scores_in=scores)
    assert np.array_equal(idx, osel.select_indices(scores, n, wl.window, wl.n_sink, k_keep))


def test_chunked_topk_identity_and_all_equal():
    n = 9000
    wl, k, v, _, cap = _tiny(n)
    s = Sel(wl, k, v, n, cap, n)
    _, idx = s.run(scores_in=np.zeros((wl.n_kv_heads, n), np.float32))
    assert np.array_equal(idx, np.tile(np.arange(n, dtype=np.int32), (wl.n_kv_heads, 1)))
    s2 = Sel(wl, k, v, n, cap, 1000)
    _, idx2 = s2.run(scores_in=np.full((wl.n_kv_heads, n), 0.5, np.float32))
    m = 1000 - wl.n_sink - wl.window
    want = list(range(wl.n_sink)) + list(range(wl.n_sink, wl.n_sink + m)) + \
        list(range(n - wl.window, n))
    assert idx2.tolist() == [want] * wl.n_kv_heads


def test_gather_copies_selected_rows_exactly():
    wl, k, v, qw, cap = _tiny()
    s = Sel(wl, k, v, 2048, cap, wl.k_keep)
    want_s = osel.window_scores(qw, k, 2048, 1 / np.sqrt(wl.head_dim)).astype(np.float32)
    _, idx = s.run(scores_in=want_s)
    want_idx = osel.select_indices(want_s, 2048, wl.window, wl.n_sink, wl.k_keep)
    assert np.array_equal(idx, want_idx)
    ks = to_host(s.ks)[:, :wl.k_keep]
    vs = to_host(s.vs)[:, :wl.k_keep]
    assert np.array_equal(ks, osel.gather(k, want_idx))
    assert np.array_equal(vs, osel.gather(v, want_idx))
    assert not to_host(s.ks)[:, wl.k_keep:].any()  # rows beyond the kept ones untouched


def test_keep_ratio_one_is_identity_copy():
    wl, k, v, qw, cap = _tiny(1500)
    s = Sel(wl, k, v, 1500, cap, 1500)
    _, idx = s.run(qw)
    assert np.array_equal(idx, np.tile(np.arange(1500, dtype=np.int32), (wl.n_kv_heads, 1)))
    assert np.array_equal(to_host(s.ks)[:, :1500], k[:, :1500])
    s2 = Sel(wl, k, v, 1500, cap, 4000)   # k_keep > n also keeps everything
    _, idx2 = s2.run(qw)
    assert idx2.shape == (wl.n_kv_heads, 1500) and np.array_equal(idx2, idx)


def test_all_equal_scores_take_lowest_candidates():
    wl, k, v, _, cap = _tiny(400)
    s = Sel(wl, k, v, 400, cap, 100)
    _, idx = s.run(scores_in=np.full((wl.n_kv_heads, 400), 0.125, np.float32))
    want = list(range(4)) + list(range(4, 68)) + list(range(368, 400))
    assert idx.tolist() == [want, want]


def test_kv_32k_planted_keys_8b():
    # the KV workload: 8B-class layer at 32K, 16% keep, 64 planted keys
    wl = synth.L8B_KV_32K
    n = wl.n_ctx
    k, v = synth.kv_cache(wl, 0, n, n)
    qw = synth.window_queries(wl, 0)
    pos = synth.plant_keys(wl, 0, k, n, qw)
    s = Sel(wl, k, v, n, n, wl.k_keep)
    got_s, got_idx = s.run(qw)
    want_s = osel.window_scores(qw, k, n, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(got_s, want_s) <= 1e-5
    for kv in range(wl.n_kv_heads):               # every planted key survives, every head
        assert set(pos.tolist()) <= set(got_idx[kv].tolist())
    want_idx = osel.select_indices(want_s.astype(np.float32), n, wl.window, wl.n_sink, wl.k_keep)
    # informational: GPU's own ranking vs the oracle's (may differ at near-ties)
    diff = sum(len(set(a) ^ set(b)) for a, b in zip(got_idx.tolist(), want_idx.tolist()))
    assert diff <= 0.001 * wl.k_keep * wl.n_kv_heads
    # bit-exact ranking and gather on the oracle's own float32 scores
    _, idx = s.run(scores_in=want_s.astype(np.float32))
    assert np.array_equal(idx, want_idx)
    kv0 = to_host(s.ks)[:, :wl.k_keep]
    assert np.array_equal(kv0, osel.gather(k, want_idx))


def test_select_is_deterministic():
    wl, k, v, qw, cap = _tiny(4096 + 37)
    s = Sel(wl, k, v, 4096 + 37, cap, 1000)
    a_s, a_i = s.run(qw)
    b_s, b_i = s.run(qw)
    assert np.array_equal(a_s, b_s) and np.array_equal(a_i, b_i)


@pytest.mark.parametrize("n,w", [(3001, 5), (2048, 32), (777, 64), (300, 1)])
def test_8b_bf16_scores_match_oracle(n, w):
    # bf16 caches score on the matrix cores (queries split into three bf16
    # parts): float32-accurate logits, ragged chunk and query-batch tails
    wl = dataclasses.replace(synth.L8B_KV_32K, n_ctx=n, window=w)
    k, v = synth.kv_cache(wl, 5, n, n + 8)
    qw = synth.window_queries(wl, 5)
    s = Sel(wl, k, v, n, n + 8, min(n, max(wl.n_sink + w, n // 4)))
    got, idx = s.run(qw)
    want = osel.window_scores(qw, k, n, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(got, want) <= 1e-5
    # each window query's softmax sums to one: G * w per KV head
    np.testing.assert_allclose(got.sum(1), 4 * w, rtol=1e-5)
    want_idx = osel.select_indices(got, n, w, wl.n_sink, s.k_keep)
    assert np.array_equal(idx, want_idx)   # the GPU ranks its own scores exactly


@pytest.mark.parametrize("h_q,h_kv,dtype,dh", [(8, 8, "bf16", 128), (64, 8, "bf16", 128),
                                               (16, 2, "f32", 64), (2, 2, "f32", 64)])
def test_query_group_sizes_scores_and_ranking(h_q, h_kv, dtype, dh):
    # one and eight query heads per KV head: the summed window scores against
    # the oracle, and the GPU's ranking of its own scores exact
    n, w = 5000, 32
    wl = dataclasses.replace(synth.L8B_KV_32K, name=f"sel-g{h_q // h_kv}-{dtype}", wid=6,
                             n_q_heads=h_q, n_kv_heads=h_kv, head_dim=dh, dtype=dtype, n_ctx=n,
                             window=w)
    k, v = synth.kv_cache(wl, 3, n, n + 8)
    qw = synth.window_queries(wl, 3)
    s = Sel(wl, k, v, n, n + 8, 1200)
    got, idx = s.run(qw)
    want = osel.window_scores(qw, k, n, 1 / np.sqrt(dh))
    assert rel_l2(got, want) <= 1e-5
    np.testing.assert_allclose(got.sum(1), (h_q // h_kv) * w, rtol=1e-5)
    assert np.array_equal(idx, osel.select_indices(got, n, w, wl.n_sink, 1200))
