"""GPU parity of the ragged per-KV-head budgets (CateKV-style hybrid retention,
"CateKV: On Sequential Consistency for Long-Context LLM Inference
Acceleration", §3 "CateKV Cache Policy"): sd_select_kv_ragged bit-exact per
head on the oracle's float32 scores, sd_decode_attn_ragged against the
float64 oracle, and decode steps over ragged gathered buffers (CATS and TEAL
projections) against the oracle's decoder layer."""

import ctypes

import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import attention as oatt, selection as osel

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import DEV, TOL, dims_for, rel_l2, to_dev, to_host, workspace  # noqa: E402
from test_gpu_step import Stack  # noqa: E402

SENTINEL = -7


class RSel:
    """Device buffers for one ragged selection call."""

    def __init__(self, wl, k, v, n, cap, k_heads, extra=4):
        self.wl, self.n, self.cap, self.k_heads = wl, n, cap, list(k_heads)
        self.k_eff = [min(x, n) for x in self.k_heads]
        self.stride = max(self.k_eff) + 3          # wider than needed: tails stay untouched
        self.cap_sel = max(self.k_eff) + extra
        self.dims = dims_for(wl)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.kd, self.vd = to_dev(k, wl.dtype), to_dev(v, wl.dtype)
        self.ks = torch.zeros(wl.n_kv_heads, self.cap_sel, wl.head_dim, dtype=tdt, device=DEV)
        self.vs = torch.zeros_like(self.ks)
        self.scores = torch.empty(wl.n_kv_heads, n, device=DEV)
        self.idx = torch.full((wl.n_kv_heads, self.stride), SENTINEL, dtype=torch.int32,
                              device=DEV)
        self.ws = workspace(self.dims, n, max(64, wl.window))

    def run(self, q_win=None, scores_in=None, w=None, n_sink=None):
        wl = self.wl
        w = wl.window if w is None else w
        n_sink = wl.n_sink if n_sink is None else n_sink
        flags, qd = 0, None
        if scores_in is not None:
            self.scores.copy_(torch.from_numpy(np.ascontiguousarray(scores_in, np.float32)))
            flags = sd.SD_SCORES_IN
        else:
            qd = to_dev(q_win)
        sd.sd_select_kv_ragged(self.dims, self.kd, self.vd, self.cap, self.n, qd, w, n_sink,
                               self.k_heads, self.scores, self.idx, self.stride, self.ks, self.vs,
                               self.cap_sel, flags, self.ws)
        torch.cuda.synchronize()
        raw = self.idx.cpu().numpy()
        return to_host(self.scores), [raw[h, :ke] for h, ke in enumerate(self.k_eff)], raw


def _tiny(n, seed_layer=0):
    wl = synth.TINY
    k, v = synth.kv_cache(wl, seed_layer, n, n + 16)
    return wl, k, v, synth.window_queries(wl, seed_layer), n + 16


@pytest.mark.parametrize("n,w,n_sink,k_heads", [
    (2048, 32, 4, [36, 2048]), (2049, 32, 4, [513, 100]), (777, 5, 0, [5, 777]),
    (300, 32, 4, [4000, 36]), (1000, 1, 1, [2, 999])])
def test_tiny_ragged_topk_and_gather_bit_exact(n, w, n_sink, k_heads):
    wl, k, v, _, cap = _tiny(n)
    scores = np.random.default_rng(n).random((wl.n_kv_heads, n)).astype(np.float32)
    s = RSel(wl, k, v, n, cap, k_heads)
    _, idx, raw = s.run(scores_in=scores, w=w, n_sink=n_sink)
    want = osel.select_indices_ragged(scores, n, w, n_sink, k_heads)
    gk, gv = to_host(s.ks), to_host(s.vs)
    for h in range(wl.n_kv_heads):
        assert np.array_equal(idx[h], want[h]), h
        assert (raw[h, len(want[h]):] == SENTINEL).all()          # tail of the row untouched
        assert np.array_equal(gk[h, :len(want[h])], osel.gather_ragged(k, want)[h])
        assert np.array_equal(gv[h, :len(want[h])], osel.gather_ragged(v, want)[h])
        assert not gk[h, len(want[h]):].any()                     # rows past the budget untouched


def test_tiny_ragged_with_window_scores_equals_uniform_per_head():
    # computed scores: each head's list equals what the uniform entry point
    # keeps with that head's budget
    wl, k, v, qw, cap = _tiny(2048)
    s = RSel(wl, k, v, 2048, cap, [100, 700])
    got_s, idx, _ = s.run(qw)
    want_s = osel.window_scores(qw, k, 2048, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(got_s, want_s) <= TOL["f32"]
    for h, kk in enumerate((100, 700)):
        u = RSel(wl, k, v, 2048, cap, [kk, kk])
        _, uidx, _ = u.run(qw)
        assert np.array_equal(idx[h], uidx[h])


def test_8b_catekv_budgets_at_32k_bit_exact():
    # the CateKV setting: 3 of 8 KV heads adaptive (eta = 1 keeps all), the
    # others keep 2048 entries
    wl = synth.L8B_KV_32K
    n = wl.n_ctx
    k, v = synth.kv_cache(wl, 0, n, n)
    qw = synth.window_queries(wl, 0)
    adaptive = [h in (1, 4, 6) for h in range(wl.n_kv_heads)]
    budgets = osel.catekv_budgets(n, adaptive, 2048, 1.0)
    s = RSel(wl, k, v, n, n, budgets)
    got_s, _, _ = s.run(qw)
    want_s = osel.window_scores(qw, k, n, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(got_s, want_s) <= 1e-5
    s32 = want_s.astype(np.float32)
    _, idx, _ = s.run(scores_in=s32)
    want = osel.select_indices_ragged(s32, n, wl.window, wl.n_sink, budgets)
    gk = to_host(s.ks)
    for h in range(wl.n_kv_heads):
        assert np.array_equal(idx[h], want[h]), h
        assert np.array_equal(gk[h, :len(want[h])], k[h, want[h]]), h


# ------------------------------------------------------------------ attention

def _attn(wl, k, v, cap, lens, q, n_splits=0):
    dims = dims_for(wl)
    kd, vd, qd = to_dev(k, wl.dtype), to_dev(v, wl.dtype), to_dev(q)
    out = torch.empty(wl.n_q_heads, wl.head_dim, device=DEV)
    lse = torch.empty(wl.n_q_heads, device=DEV)
    sd.sd_decode_attn_ragged(dims, qd, kd, vd, cap, lens, 1 / np.sqrt(wl.head_dim), n_splits, out,
                             lse, workspace(dims))
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


@pytest.mark.parametrize("lens,splits", [([1, 2048], 0), ([2049, 1], 0), ([300, 4099], 17),
                                         ([4099, 129], 128), ([64, 64], 64), ([5, 3000], 7),
                                         ([4099, 129], 256), ([70000, 3000], 0),
                                         ([2000, 40000], 200)])
def test_tiny_fp32_ragged_attention_matches_oracle(lens, splits):
    wl = synth.TINY
    cap = max(lens) + 8
    k, v = synth.kv_cache(wl, 1, cap, cap)
    q = synth.decode_query(wl, 1)
    out, lse = _attn(wl, k, v, cap, lens, q, splits)
    want, wlse = oatt.attend_ragged(q, k, v, lens, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(out, want) <= TOL["f32"]
    np.testing.assert_allclose(lse, wlse, rtol=1e-5, atol=1e-5)


def test_equal_lengths_reproduce_the_uniform_kernel_bitwise():
    wl = synth.L8B_DENSE_8K
    n = 5000
    k, v = synth.kv_cache(wl, 2, n, n)
    q = synth.decode_query(wl, 2)
    out, lse = _attn(wl, k, v, n, [n] * wl.n_kv_heads, q)
    dims = dims_for(wl)
    uo = torch.empty(wl.n_q_heads, wl.head_dim, device=DEV)
    ul = torch.empty(wl.n_q_heads, device=DEV)
    sd.sd_decode_attn(dims, to_dev(q), to_dev(k, wl.dtype), to_dev(v, wl.dtype), n, n,
                      1 / np.sqrt(wl.head_dim), 0, uo, ul, workspace(dims))
    torch.cuda.synchronize()
    assert np.array_equal(out, to_host(uo)) and np.array_equal(lse, to_host(ul))


def test_8b_bf16_catekv_lengths_match_oracle():
    wl = synth.L8B_KV_32K
    n = wl.n_ctx
    adaptive = [h in (1, 4, 6) for h in range(wl.n_kv_heads)]
    lens = osel.catekv_budgets(n, adaptive, 2048, 1.0)
    k, v = synth.kv_cache(wl, 3, n, n)
    q = synth.decode_query(wl, 3)
    out, lse = _attn(wl, k, v, n, lens, q)
    want, wlse = oatt.attend_ragged(q, k, v, lens, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(out, want) <= TOL["bf16"]
    np.testing.assert_allclose(lse, wlse, rtol=1e-4, atol=1e-4)


# ------------------------------------------------------------------ the step

class RaggedStack(Stack):
    """Stack whose gathered buffers hold ragged per-head selections."""

    def __init__(self, wl, n_layers, n, adaptive, budget, extra=8, **kw):
        super().__init__(wl, n_layers, n, budget, extra=extra, **kw)
        self.heads_host = []
        for li in range(n_layers):
            ol = self.olayers[li]
            qw = synth.window_queries(wl, li)
            s32 = osel.window_scores(qw, ol.k_full, n, 1 / np.sqrt(wl.head_dim)).astype(np.float32)
            kh = osel.catekv_budgets(n, adaptive, budget, 1.0)
            idx = osel.select_indices_ragged(s32, n, wl.window, wl.n_sink, kh)
            cap_sel = max(len(x) for x in idx) + extra
            ks = np.zeros((wl.n_kv_heads, cap_sel, wl.head_dim), np.float32)
            vs = np.zeros_like(ks)
            for h, ix in enumerate(idx):
                ks[h, :len(ix)] = ol.k_full[h, ix]
                vs[h, :len(ix)] = ol.v_full[h, ix]
            ol.k_sel, ol.v_sel = ks.astype(np.float64), vs.astype(np.float64)
            ol.n_sel_heads = [len(x) for x in idx]
            dks, dvs = to_dev(ks, wl.dtype), to_dev(vs, wl.dtype)
            heads = (ctypes.c_int32 * wl.n_kv_heads)(*ol.n_sel_heads)
            self.heads_host.append(heads)
            self.keep_alive[li] = self.keep_alive[li][:3] + (dks, dvs) + self.keep_alive[li][5:]
            L = self.layers[li]
            L.k_sel, L.v_sel, L.cap_sel = dks.data_ptr(), dvs.data_ptr(), cap_sel
            L.n_sel_heads = heads


def _check_ragged_caches(st, tol):
    for li, ol in enumerate(st.olayers):
        dks = st.keep_alive[li][3]
        assert list(st.heads_host[li]) == ol.n_sel_heads
        g = to_host(dks)
        for h, m in enumerate(ol.n_sel_heads):
            assert rel_l2(g[h, :m], ol.k_sel[h, :m]) <= tol
            assert not g[h, m:].any()


def test_tiny_fp32_ragged_steps_with_mode_switching():
    wl = synth.TINY
    st = RaggedStack(wl, 1, wl.n_ctx, [False, True], 300, extra=16)
    h = synth.hidden(wl, 0).astype(np.float64)
    pos = wl.n_ctx
    for mode in ("kv", "both", "dense", "kv", "cats", "both"):
        got, want, _ = st.step(h, pos, mode)
        assert rel_l2(got, want) <= TOL["f32"], mode
        h = want
        pos += 1
    assert st.olayers[0].n_sel_heads == [300 + 6, wl.n_ctx + 6]
    _check_ragged_caches(st, TOL["f32"])


def test_8b_ragged_two_layers_both():
    wl = synth.L8B_DENSE_8K
    adaptive = [h in (1, 4, 6) for h in range(wl.n_kv_heads)]
    st = RaggedStack(wl, 2, 4096, adaptive, 512)
    h = synth.hidden(wl, 3)
    pos = 4096
    for mode in ("kv", "both"):
        got, want, _ = st.step(h, pos, mode)
        assert rel_l2(got, want) <= TOL["bf16"], mode
        h = want
        pos += 1
    _check_ragged_caches(st, TOL["bf16"])


def test_tiny_fp32_ragged_teal_step():
    # TEAL projections over a ragged gathered buffer: the QKV epilogue appends
    # each KV head at its own row
    from test_gpu_teal import TealStack

    class RTeal(RaggedStack):
        add_teal = TealStack.add_teal
        thresholds = TealStack.thresholds
        teal_step = TealStack.teal_step

    wl = synth.TINY
    st = RTeal(wl, 1, wl.n_ctx, [True, False], 200, extra=16)
    st.add_teal(wl, 1)
    h = synth.hidden(wl, 2).astype(np.float64)
    got, want, tr, gm = st.teal_step(h, wl.n_ctx, kv_sparse=True)
    assert rel_l2(got, want) <= TOL["f32"]
    assert st.olayers[0].n_sel_heads == [wl.n_ctx + 1, 201]
    _check_ragged_caches(st, TOL["f32"])


@pytest.mark.parametrize("h_q,h_kv", [(8, 8), (64, 8)])
@pytest.mark.parametrize("splits", [0, 256])
def test_ragged_attention_group_sizes_match_oracle(h_q, h_kv, splits):
    # one and eight query heads per KV head over per-head lengths from one
    # row to 20001 (bf16, d_h 128)
    wl = dataclasses.replace(synth.L8B_DENSE_8K, name=f"ragged-g{h_q // h_kv}", wid=6,
                             n_q_heads=h_q, n_kv_heads=h_kv)
    lens = [1, 20001, 300, 4099, 64, 12000, 2, 777]
    cap = max(lens) + 8
    k, v = synth.kv_cache(wl, 1, cap, cap)
    q = synth.decode_query(wl, 1)
    out, lse = _attn(wl, k, v, cap, lens, q, splits)
    want, wlse = oatt.attend_ragged(q, k, v, lens, 1 / np.sqrt(wl.head_dim))
    assert rel_l2(out, want) <= TOL["bf16"]
    assert rel_l2(lse, wlse) <= TOL["bf16"]
