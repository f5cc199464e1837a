"""GPU parity of sd_decode_step_batch (B sequences sharing every weight read,
union channel masks; "Where Activation Sparsity and KV-Cache Sparsity Cross
in LLM Decoding", §3.3 "Dispatch and batching", §4.4 "Batching") against the
float64 batch oracle: every sequence's new hidden state, the union mask bit
for bit, and the appended cache rows."""

import copy
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import batch as obatch, selection as osel, step as ostep

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import (DEV, TOL, dims_for, midpoint_threshold, rel_l2, to_dev,  # noqa: E402
                         to_host)

MODES = {"dense": 0, "kv": sd.SD_KV_SPARSE, "cats": sd.SD_MLP_SPARSE,
         "both": sd.SD_KV_SPARSE | sd.SD_MLP_SPARSE}


class BatchStack:
    """B sequences over shared layer weights: each sequence has its own caches
    (its own context length) and its own gathered buffer from the oracle's
    selection."""

    def __init__(self, wl, n_layers, batch, n, keep_ratio, extra=8, matrix_cores=False,
                 kv_dtype=None):
        self.wl, self.B, self.L = wl, batch, n_layers
        self.mc = matrix_cores
        kvt = kv_dtype or wl.dtype   # the caches' type (the weights' by default)
        self.dims = dims_for(wl)
        self.dims.kv_dtype = sd.SD_BF16 if kvt == "bf16" else sd.SD_F32
        self.odims = dict(n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                          head_dim=wl.head_dim, kv_dtype=kvt, eps=1e-5, theta=500000.0)
        self.keep_alive = []
        W = [synth.layer_weights(wl, li) for li in range(n_layers)]
        layers = []
        for li in range(n_layers):
            dW = {k: to_dev(v, "f32" if "norm" in k else wl.dtype) for k, v in W[li].items()}
            mask = torch.zeros(wl.d_ff, dtype=torch.uint8, device=DEV)
            self.keep_alive.append((dW, mask))
            layers.append(sd.sd_layer(dW["attn_norm"].data_ptr(), dW["w_qkv"].data_ptr(),
                                      dW["w_o"].data_ptr(), dW["mlp_norm"].data_ptr(),
                                      dW["w_gate"].data_ptr(), dW["w_up"].data_ptr(),
                                      dW["w_down_t"].data_ptr(), -1.0, 0, None, None, 0, 0,
                                      None, None, 0, 0, mask.data_ptr()))
            if matrix_cores:   # the tile weights, packed by the library
                for f, w in (("w_qkv_m", dW["w_qkv"]), ("w_o_m", dW["w_o"]),
                             ("w_gate_m", dW["w_gate"]), ("w_up_m", dW["w_up"]),
                             ("w_down_m", dW["w_down_t"].t().contiguous())):
                    t = torch.empty(sd.sd_tile_bytes(*w.shape), dtype=torch.uint8, device=DEV)
                    sd.sd_pack_tiles(w, w.shape[0], w.shape[1], t)
                    self.keep_alive.append(t)
                    setattr(layers[-1], f, t.data_ptr())
        self.layers = (sd.sd_layer * n_layers)(*layers)
        self.n = [n - 3 * b for b in range(batch)]       # a different length per sequence
        self.seq, kvs, self.dev_kv = [], [], []
        for b in range(batch):
            nb = self.n[b]
            cap = nb + extra
            k_keep = max(wl.n_sink + wl.window, int(keep_ratio * nb))
            seq = []
            for li in range(n_layers):
                seed = li + 100 * (b + 1)
                k, v = synth.kv_cache(wl, seed, nb, cap)
                qw = synth.window_queries(wl, seed)
                s32 = osel.window_scores(qw, k, nb, 1 / np.sqrt(wl.head_dim)).astype(np.float32)
                idx = osel.select_indices(s32, nb, wl.window, wl.n_sink, k_keep)
                ke = idx.shape[1]
                ks = np.zeros((wl.n_kv_heads, ke + extra, wl.head_dim), np.float32)
                vs = np.zeros_like(ks)
                ks[:, :ke] = osel.gather(k, idx)
                vs[:, :ke] = osel.gather(v, idx)
                w = W[li]
                seq.append(ostep.Layer(w["attn_norm"], w["w_qkv"], w["w_o"], w["mlp_norm"],
                                       w["w_gate"], w["w_up"], w["w_down_t"], -1.0, k, v, nb,
                                       ks, vs, ke))
                dk, dv, dks, dvs = (to_dev(a, kvt) for a in (k, v, ks, vs))
                self.dev_kv.append((dk, dv, dks, dvs))
                kvs.append(sd.sd_seq_kv(dk.data_ptr(), dv.data_ptr(), cap, nb, dks.data_ptr(),
                                        dvs.data_ptr(), ke + extra, ke))
            self.seq.append(seq)
        self.kv = (sd.sd_seq_kv * (batch * n_layers))(*kvs)
        self.ws = torch.empty(sd.sd_batch_workspace_bytes(self.dims, batch), dtype=torch.uint8,
                              device=DEV)

    def thresholds(self, hs, pos, sparsity, kv_sparse):
        """Per layer one midpoint threshold over all sequences' gate
        activations (each layer's inputs follow the earlier layers' masks)."""
        work = copy.deepcopy(self.seq)
        hh = [np.asarray(h, np.float64) for h in hs]
        ts = []
        for li in range(self.L):
            acts = []
            for b in range(self.B):
                tr = []
                ostep.decode_layer(copy.deepcopy(work[b][li]), hh[b], pos[b], kv_sparse=kv_sparse,
                                   mlp_sparse=False, trace=tr, **self.odims)
                acts.append(tr[0]["act"])
            t = midpoint_threshold(np.concatenate(acts), sparsity)
            for b in range(self.B):
                work[b][li].threshold = t
                hh[b] = ostep.decode_layer(work[b][li], hh[b], pos[b], kv_sparse=kv_sparse,
                                           mlp_sparse=True, **self.odims)
            ts.append(t)
        return ts

    def step(self, hs, pos, mode, sparsity=0.5):
        kv_sparse = bool(MODES[mode] & sd.SD_KV_SPARSE)
        mlp_sparse = bool(MODES[mode] & sd.SD_MLP_SPARSE)
        if mlp_sparse:
            for li, t in enumerate(self.thresholds(hs, pos, sparsity, kv_sparse)):
                self.layers[li].cats_threshold = t
                for b in range(self.B):
                    self.seq[b][li].threshold = t
        tr = []
        want, unions = obatch.decode_step_batch(self.seq, hs, pos, kv_sparse=kv_sparse,
                                                mlp_sparse=mlp_sparse, trace=tr, **self.odims)
        hd = to_dev(np.stack(hs))
        flags = MODES[mode] | (sd.SD_MATRIX_CORES if self.mc else 0)
        sd.sd_decode_step_batch(self.dims, self.layers, self.kv, pos, hd, flags, self.ws)
        torch.cuda.synchronize()
        got_unions = [e[1].cpu().numpy().astype(bool) for e in self.keep_alive
                      if isinstance(e, tuple)]
        return to_host(hd), want, unions, got_unions


def _check_appends(st, tol):
    for b in range(st.B):
        for li in range(st.L):
            ol = st.seq[b][li]
            kv = st.kv[b * st.L + li]
            assert kv.n_full == ol.n and kv.n_sel == ol.n_sel
            dk, dv, dks, dvs = st.dev_kv[b * st.L + li]
            assert rel_l2(to_host(dk)[:, ol.n - 1], ol.k_full[:, ol.n - 1]) <= tol
            assert rel_l2(to_host(dvs)[:, ol.n_sel - 1], ol.v_sel[:, ol.n_sel - 1]) <= tol


@pytest.mark.parametrize("batch", [2, 3, 4, 8])
def test_tiny_fp32_batch_modes_over_steps(batch):
    wl = synth.TINY
    st = BatchStack(wl, 2, batch, 600, 0.25, extra=8)
    hs = [synth.hidden(wl, 10 + b).astype(np.float64) for b in range(batch)]
    pos = list(st.n)
    for mode in ("dense", "both", "kv", "cats"):
        got, want, unions, gu = st.step(hs, pos, mode)
        for b in range(batch):
            assert rel_l2(got[b], want[b]) <= TOL["f32"], (mode, b)
        if MODES[mode] & sd.SD_MLP_SPARSE:
            for li in range(st.L):
                assert np.array_equal(gu[li], unions[li]), (mode, li)
        else:
            assert all(u.all() for u in gu)
        hs = [w for w in want]
        pos = [p + 1 for p in pos]
    _check_appends(st, TOL["f32"])


@pytest.mark.parametrize("batch", [2, 4, 8])
def test_8b_bf16_batch_both(batch):
    wl = synth.L8B_DENSE_8K
    st = BatchStack(wl, 1, batch, 2048, 0.16)
    hs = [synth.hidden(wl, 20 + b) for b in range(batch)]
    got, want, unions, gu = st.step(hs, list(st.n), "both")
    for b in range(batch):
        assert rel_l2(got[b], want[b]) <= TOL["bf16"], b
    assert np.array_equal(gu[0], unions[0])
    # independent-looking masks at 50% sparsity: the union is near 1 - 0.5^B
    u = gu[0].mean()
    assert abs(u - (1 - 0.5 ** batch)) < 0.03, u
    _check_appends(st, TOL["bf16"])


def test_8b_bf16_batch_dense_two_layers_over_steps():
    wl = synth.L8B_DENSE_8K
    st = BatchStack(wl, 2, 3, 1024, 0.2)
    hs = [synth.hidden(wl, 40 + b) for b in range(3)]
    pos = list(st.n)
    for mode in ("dense", "kv"):
        got, want, _, gu = st.step(hs, pos, mode)
        for b in range(3):
            assert rel_l2(got[b], want[b]) <= TOL["bf16"], (mode, b)
        assert all(u.all() for u in gu)
        hs = [w for w in want]
        pos = [p + 1 for p in pos]


def test_batch_matches_single_sequence_steps():
    # the batched kernels against the single-sequence path on the same inputs
    wl = synth.TINY
    st = BatchStack(wl, 1, 3, 500, 0.3)
    hs = [synth.hidden(wl, 30 + b) for b in range(3)]
    single = []
    for b in range(3):
        one = copy.deepcopy(st.seq[b])
        single.append(ostep.decode_step(one, hs[b], st.n[b], kv_sparse=True, mlp_sparse=False,
                                        **st.odims))
    got, want, _, _ = st.step(hs, list(st.n), "kv")
    for b in range(3):
        assert rel_l2(got[b], single[b]) <= TOL["f32"]
        assert np.array_equal(want[b], single[b])


def test_batch_rejections_leave_state_untouched():
    wl = synth.TINY
    st = BatchStack(wl, 1, 2, 300, 0.3)
    hd = to_dev(np.stack([synth.hidden(wl, 0), synth.hidden(wl, 1)]))
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step_batch(st.dims, st.layers, st.kv, st.n, hd, sd.SD_KV_WINDOW, st.ws)
    assert e.value.status == sd.SD_EINVAL
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step_batch(st.dims, st.layers, st.kv, st.n, hd, 0, small)
    assert e.value.status == sd.SD_ENOSPC
    assert st.kv[0].n_full == st.n[0] and st.kv[1].n_full == st.n[1]


def test_more_sequence_heads_than_split_workgroups():
    # 5 sequences x 64 KV heads (one query head each) = 320 (sequence, head)
    # pairs, more than the 256 chunk workgroups the planner aims for: every
    # pair gets one chunk and the grid has one workgroup per pair
    from dataclasses import replace
    wl = replace(synth.TINY, name="g1-64kv-heads", d_model=4096, n_q_heads=64, n_kv_heads=64,
                 head_dim=64, d_ff=1024)
    batch = 5
    st = BatchStack(wl, 1, batch, 200, 0.5)
    hs = [synth.hidden(wl, 50 + b) for b in range(batch)]
    pos = list(st.n)
    for mode in ("dense", "kv"):
        got, want, _, _ = st.step(hs, pos, mode)
        for b in range(batch):
            assert rel_l2(got[b], want[b]) <= TOL["f32"], (mode, b)
        hs = [w for w in want]
        pos = [p + 1 for p in pos]
    _check_appends(st, TOL["f32"])


# ---------------------------------------------------------------- matrix cores
# Widths that are not multiples of the 16-row tiles or the 32-channel steps:
# O and down have 264 output rows (16.5 tiles), QKV and gate/up read 264
# input channels (8.25 steps), down reads 680 (21.25 steps), gate/up have
# 680 rows.
RAGGED_BF16 = replace(synth.TINY, name="ragged-bf16-2layer", wid=9, d_model=264, d_ff=680,
                      dtype="bf16")


def test_pack_tiles_is_the_documented_relayout():
    from synth import device as sdev
    g = torch.Generator().manual_seed(5)
    for rows, d_in in ((40, 200), (16, 32), (6144 // 8, 4096 // 8)):
        w = torch.randn(rows, d_in, generator=g).to(torch.bfloat16).to(DEV)
        out = torch.full((sd.sd_tile_bytes(rows, d_in),), 0xAB, dtype=torch.uint8, device=DEV)
        sd.sd_pack_tiles(w, rows, d_in, out)
        torch.cuda.synchronize()
        want = sdev.mma_tiles(w).view(torch.uint8).flatten()
        assert torch.equal(out, want), (rows, d_in)
    # element (r, c) sits where the header says
    rows, d_in = 40, 200
    w = torch.arange(rows * d_in, dtype=torch.float32).remainder(251).to(torch.bfloat16)
    w = w.view(rows, d_in).to(DEV)
    out = torch.empty(sd.sd_tile_bytes(rows, d_in), dtype=torch.uint8, device=DEV)
    sd.sd_pack_tiles(w, rows, d_in, out)
    flat = out.view(torch.bfloat16).cpu()
    T = (rows + 15) // 16
    for r, c in ((0, 0), (17, 33), (39, 199), (5, 100), (31, 64)):
        i = ((c // 32) * T + r // 16) * 512 + ((r % 16) + 16 * ((c % 32) // 8)) * 8 + c % 8
        assert flat[i] == w[r, c].cpu(), (r, c)


@pytest.mark.parametrize("batch", [2, 3, 5, 8])
def test_matrix_cores_ragged_widths_modes_over_steps(batch):
    wl = RAGGED_BF16
    st = BatchStack(wl, 2, batch, 600, 0.25, extra=8, matrix_cores=True)
    hs = [synth.hidden(wl, 10 + b).astype(np.float64) for b in range(batch)]
    pos = list(st.n)
    for mode in ("dense", "both", "kv", "cats"):
        got, want, unions, gu = st.step(hs, pos, mode)
        for b in range(batch):
            assert rel_l2(got[b], want[b]) <= TOL["bf16"], (mode, b)
        if MODES[mode] & sd.SD_MLP_SPARSE:
            for li in range(st.L):
                assert np.array_equal(gu[li], unions[li]), (mode, li)
        else:
            assert all(u.all() for u in gu)
        hs = [w for w in want]
        pos = [p + 1 for p in pos]
    _check_appends(st, TOL["bf16"])


@pytest.mark.parametrize("batch", [2, 4, 8])
def test_matrix_cores_8b_bf16_batch_both(batch):
    wl = synth.L8B_DENSE_8K
    st = BatchStack(wl, 1, batch, 2048, 0.16, matrix_cores=True)
    hs = [synth.hidden(wl, 20 + b) for b in range(batch)]
    got, want, unions, gu = st.step(hs, list(st.n), "both")
    for b in range(batch):
        assert rel_l2(got[b], want[b]) <= TOL["bf16"], b
    assert np.array_equal(gu[0], unions[0])
    _check_appends(st, TOL["bf16"])


def test_matrix_cores_8b_two_layers_dense_then_cats():
    wl = synth.L8B_DENSE_8K
    st = BatchStack(wl, 2, 8, 1024, 0.2, matrix_cores=True)
    hs = [synth.hidden(wl, 60 + b) for b in range(8)]
    pos = list(st.n)
    for mode in ("dense", "cats"):
        got, want, unions, gu = st.step(hs, pos, mode)
        for b in range(8):
            assert rel_l2(got[b], want[b]) <= TOL["bf16"], (mode, b)
        if mode == "cats":
            for li in range(2):
                assert np.array_equal(gu[li], unions[li]), li
        hs = [w for w in want]
        pos = [p + 1 for p in pos]


# 128-dim heads: each 128-row group of W_qkv is one head, so the matrix-core
# QKV applies RoPE and the appends in its epilogue (bf16 caches; float32
# caches keep the separate RoPE launch), and O merges the attention's split
# partials while staging its input.
HEAD128_BF16 = replace(synth.TINY, name="head128-bf16-2layer", wid=10, d_model=512, n_q_heads=4,
                       n_kv_heads=2, head_dim=128, d_ff=1024, dtype="bf16")


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("batch", [2, 3, 5, 8])
def test_matrix_cores_head128_fused_epilogues_modes_over_steps(batch, kv_dtype):
    wl = HEAD128_BF16
    st = BatchStack(wl, 2, batch, 600, 0.25, extra=8, matrix_cores=True, kv_dtype=kv_dtype)
    hs = [synth.hidden(wl, 30 + b).astype(np.float64) for b in range(batch)]
    pos = list(st.n)
    for mode in ("both", "dense", "kv", "cats"):
        got, want, unions, gu = st.step(hs, pos, mode)
        for b in range(batch):
            assert rel_l2(got[b], want[b]) <= TOL["bf16"], (mode, b)
        if MODES[mode] & sd.SD_MLP_SPARSE:
            for li in range(st.L):
                assert np.array_equal(gu[li], unions[li]), (mode, li)
        hs = [w for w in want]
        pos = [p + 1 for p in pos]
    _check_appends(st, TOL["bf16"])
