"""GPU parity of sd_teal_gemv (one TEAL-sparse projection: |x| > t on the input,
only the kept input channels' weight rows read) and of the SD_PROJ_TEAL decode
step (all seven projections) against the float64 TEAL oracle."""

import copy
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import teal as oteal, step as ostep

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import (DEV, TOL, dims_for, midpoint_threshold, rel_l2, teal_dev, to_dev,  # noqa
                         to_host, workspace)
from test_gpu_step import Stack  # noqa: E402


def _weight_t(rng, d_in, d_out, dtype):
    w = (rng.standard_normal((d_in, d_out)) * 0.02).astype(np.float32)
    return synth.to_bf16_values(w) if dtype == "bf16" else w


class Gemv:
    def __init__(self, wl, d_in, d_out, dual=False, seed=0):
        self.wl, self.d_in, self.d_out = wl, d_in, d_out
        self.dims = dims_for(wl)
        r = np.random.default_rng(seed)
        self.wt = _weight_t(r, d_in, d_out, wl.dtype)
        self.wt2 = _weight_t(r, d_in, d_out, wl.dtype) if dual else None
        self.norm = (1.0 + 0.1 * r.standard_normal(d_in)).astype(np.float32)
        # the device copies in the column-block layout of W = wt^T
        self.dw = teal_dev(self.wt.T, wl.dtype)
        self.dw2 = teal_dev(self.wt2.T, wl.dtype) if dual else None
        self.y = torch.empty(d_out, device=DEV)
        self.y2 = torch.empty(d_out, device=DEV) if dual else None
        self.idx = torch.empty(d_in, dtype=torch.int32, device=DEV)
        self.nk = torch.empty(1, dtype=torch.int32, device=DEV)
        self.ws = workspace(self.dims)

    def run(self, x, t, norm=False, flags=0, y0=None):
        if y0 is not None:
            self.y.copy_(torch.from_numpy(y0))
            if self.y2 is not None:
                self.y2.copy_(torch.from_numpy(y0))
        sd.sd_teal_gemv(self.dims, to_dev(x), self.d_in, to_dev(self.norm) if norm else None, t,
                        self.dw, self.dw2, self.d_out, self.y, self.y2, flags, self.idx, self.nk,
                        self.ws)
        torch.cuda.synchronize()
        nk = int(self.nk.item())
        y2 = to_host(self.y2) if self.y2 is not None else None
        return to_host(self.y), y2, self.idx.cpu().numpy()[:nk]

    def xhat(self, x, norm):
        return ostep.rmsnorm(x, self.norm, 1e-5) if norm else np.asarray(x, np.float64)


CASES = [(synth.TINY, 256, 688), (synth.TINY, 688, 256), (synth.TINY, 264, 72),
         (synth.L8B_DENSE_8K, 4096, 6144), (synth.L8B_DENSE_8K, 4096, 4096),
         (synth.L8B_DENSE_8K, 14336, 4096), (synth.L8B_DENSE_8K, 4104, 4104)]


@pytest.mark.parametrize("wl,d_in,d_out", CASES, ids=lambda c: getattr(c, "name", str(c)))
@pytest.mark.parametrize("sparsity", [None, 0.5, 0.9])
@pytest.mark.parametrize("norm", [False, True])
def test_teal_gemv_matches_oracle(wl, d_in, d_out, sparsity, norm):
    g = Gemv(wl, d_in, d_out, seed=d_in + d_out)
    x = np.random.default_rng(d_in).standard_normal(d_in).astype(np.float32)
    xh = g.xhat(x, norm)
    # a midpoint threshold leaves half a gap between it and every |x_hat|, so
    # float32 rounding of the norm cannot flip a channel: masks match exactly
    t = -1.0 if sparsity is None else midpoint_threshold(xh, sparsity)
    y, _, idx = g.run(x, t, norm)
    want, mask, widx = oteal.teal_linear(g.wt.T, xh, t)
    assert np.array_equal(idx, widx)
    if sparsity is not None:
        assert idx.size == d_in - int(np.floor(sparsity * d_in + 0.5))
    assert rel_l2(y, want) <= TOL[wl.dtype]


def test_teal_gemv_threshold_is_strict_on_exact_ties():
    # no norm: both sides decide on the same float32 inputs, entries exactly at
    # +-t are dropped and one ulp above is kept
    wl = synth.TINY
    g = Gemv(wl, 256, 688)
    x = np.random.default_rng(3).standard_normal(256).astype(np.float32)
    t = np.float32(0.5)
    x[:4] = [t, -t, np.nextafter(t, np.float32(1)), -np.nextafter(t, np.float32(1))]
    y, _, idx = g.run(x, float(t))
    want, mask, widx = oteal.teal_linear(g.wt.T, x, float(t))
    assert 0 not in idx and 1 not in idx and 2 in idx and 3 in idx
    assert np.array_equal(idx, widx)
    assert rel_l2(y, want) <= TOL["f32"]


def test_teal_gemv_dual_accumulate_and_all_dropped():
    wl = synth.L8B_DENSE_8K
    g = Gemv(wl, 4096, 14336, dual=True, seed=5)
    x = np.random.default_rng(6).standard_normal(4096).astype(np.float32)
    y0 = np.random.default_rng(7).standard_normal(14336).astype(np.float32)
    t = midpoint_threshold(x, 0.5)
    y, y2, idx = g.run(x, t, flags=sd.SD_ACCUMULATE, y0=y0)
    w1, mask, widx = oteal.teal_linear(g.wt.T, x, t)
    w2 = oteal.linear_masked(g.wt2.T, x, mask)
    assert np.array_equal(idx, widx)
    assert rel_l2(y - y0, w1) <= TOL["bf16"] and rel_l2(y2 - y0, w2) <= TOL["bf16"]
    # nothing kept: the result is exactly zero (or y unchanged when accumulating)
    y, y2, idx = g.run(x, 1e9)
    assert idx.size == 0 and not y.any() and not y2.any()
    y, _, idx = g.run(x, 1e9, flags=sd.SD_ACCUMULATE, y0=y0)
    assert np.array_equal(y, y0)


def test_teal_gemv_is_deterministic():
    wl = synth.L8B_DENSE_8K
    g = Gemv(wl, 14336, 4096, seed=8)
    x = np.random.default_rng(9).standard_normal(14336).astype(np.float32)
    t = midpoint_threshold(x, 0.5)
    a = g.run(x, t)[0]
    b = g.run(x, t)[0]
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ the step

class TealStack(Stack):
    """Stack plus the column-block weights and the mask buffers of SD_PROJ_TEAL."""

    def __init__(self, wl, n_layers, n, k_keep, **kw):
        super().__init__(wl, n_layers, n, k_keep, **kw)
        self.add_teal(wl, n_layers)

    def add_teal(self, wl, n_layers):
        self.teal_keep = []
        d, qd, ff = wl.d_model, wl.n_q_heads * wl.head_dim, wl.d_ff
        self.mask_sizes = (d, qd, d, ff)
        for li in range(n_layers):
            W = synth.layer_weights(wl, li)
            dt = {k: teal_dev(W[k], wl.dtype) for k in ("w_qkv", "w_o", "w_gate", "w_up")}
            masks = torch.zeros(sum(self.mask_sizes), dtype=torch.uint8, device=DEV)
            self.teal_keep.append((dt, masks))
            L = self.layers[li]
            L.w_qkv_t = dt["w_qkv"].data_ptr()
            L.w_o_t = dt["w_o"].data_ptr()
            L.w_gate_t = dt["w_gate"].data_ptr()
            L.w_up_t = dt["w_up"].data_ptr()
            L.teal_masks_out = masks.data_ptr()

    def thresholds(self, h, pos, kv_sparse, sparsity):
        """Per layer, the four midpoint thresholds chosen one input at a time
        from the oracle's own activations (each input depends on the earlier
        ones' masks); the oracle layers are left untouched."""
        work = copy.deepcopy(self.olayers)
        hh = np.asarray(h, np.float64)
        out = []
        for layer in work:
            ts = [-1.0] * 4
            for k, key in enumerate(("x", "attn", "x2", "hmid")):
                tr = []
                oteal.teal_layer(copy.deepcopy(layer), hh, pos, ts, kv_sparse=kv_sparse, trace=tr,
                                 **self.odims)
                ts[k] = midpoint_threshold(tr[0][key], sparsity)
            out.append(tuple(ts))
            hh = oteal.teal_layer(layer, hh, pos, ts, kv_sparse=kv_sparse, **self.odims)
        return out

    def teal_step(self, h, pos, kv_sparse, sparsity=0.5, inject=False):
        ts = self.thresholds(h, pos, kv_sparse, sparsity)
        for li, t4 in enumerate(ts):
            for k in range(4):
                self.layers[li].teal_t[k] = t4[k]
        hd = to_dev(h)
        mode = sd.SD_PROJ_TEAL | (sd.SD_KV_SPARSE if kv_sparse else 0)
        sd.sd_decode_step(self.dims, self.layers, pos, hd, mode, self.ws)
        torch.cuda.synchronize()
        gmasks = []
        for li in range(len(self.olayers)):
            raw = self.teal_keep[li][1].cpu().numpy().astype(bool)
            cut = np.cumsum((0,) + self.mask_sizes)
            gmasks.append([raw[cut[k]:cut[k + 1]] for k in range(4)])
        tr = []
        want = oteal.teal_step(self.olayers, h, pos, ts, kv_sparse=kv_sparse, trace=tr,
                               masks=gmasks if inject else None, **self.odims)
        return to_host(hd), want, tr, gmasks


@pytest.mark.parametrize("blocked_down", [False, True])
def test_tiny_fp32_teal_step_with_mode_switching(blocked_down):
    # blocked_down: the down projection over column blocks (w_down_b)
    wl = synth.TINY
    st = TealStack(wl, 1, wl.n_ctx, wl.k_keep, extra=16, blocked_down=blocked_down)
    h = synth.hidden(wl, 0).astype(np.float64)
    pos = wl.n_ctx
    from test_gpu_step import MODES
    for mode in ("teal", "teal+kv", "dense", "teal", "both"):
        if mode.startswith("teal"):
            got, want, tr, gm = st.teal_step(h, pos, kv_sparse=mode == "teal+kv")
            for k in range(4):
                assert np.array_equal(gm[0][k], tr[0]["masks"][k]), (mode, k)
                frac = gm[0][k].mean()
                assert 0.45 < frac < 0.55, (mode, k, frac)
        else:
            got, want, tr = st.step(h, pos, mode)
        assert rel_l2(got, want) <= TOL["f32"], mode
        h = want
        pos += 1


def test_tiny_fp32_teal_two_layers_dense_limit_matches_dense():
    # all four thresholds < 0: the TEAL kernels read every row and the step
    # matches the oracle's dense layer
    wl = synth.TINY
    st = TealStack(wl, 2, 1000, 300)
    h = synth.hidden(wl, 5)
    for li in range(2):
        for k in range(4):
            st.layers[li].teal_t[k] = -1.0
    hd = to_dev(h)
    sd.sd_decode_step(st.dims, st.layers, 1000, hd, sd.SD_PROJ_TEAL, st.ws)
    torch.cuda.synchronize()
    want = ostep.decode_step(st.olayers, h, 1000, kv_sparse=False, mlp_sparse=False, **st.odims)
    assert rel_l2(to_host(hd), want) <= TOL["f32"]
    for li in range(2):
        assert st.teal_keep[li][1].cpu().numpy().all()


@pytest.mark.parametrize("n_q,n_kv,n", [(4, 1, 2400), (8, 2, 5000), (4, 1, 16383)])
def test_tiny_fp32_teal_step_head_groups_and_split_counts(n_q, n_kv, n):
    """The TEAL step with four query heads per KV head and dense steps of 38,
    79 and 256 attention splits, KV steps of 10, 20 and 64."""
    wl = dataclasses.replace(synth.TINY, name=f"tiny-f32-h{n_q}x{n_kv}", n_q_heads=n_q,
                             n_kv_heads=n_kv, n_ctx=n)
    st = TealStack(wl, 1, n, n // 4, extra=8, blocked_down=True)
    h = synth.hidden(wl, 6).astype(np.float64)
    pos = n
    for kv_sparse in (False, True):
        got, want, tr, gm = st.teal_step(h, pos, kv_sparse)
        assert rel_l2(got, want) <= TOL["f32"], kv_sparse
        for k in range(4):
            assert np.array_equal(gm[0][k], tr[0]["masks"][k]), (kv_sparse, k)
        h = want
        pos += 1


@pytest.mark.parametrize("blocked_down", [False, True])
@pytest.mark.parametrize("kv_sparse", [False, True])
def test_8b_teal_layer_matches_oracle_with_its_masks(kv_sparse, blocked_down):
    wl = synth.L8B_DENSE_8K
    st = TealStack(wl, 1, 4096, 655, blocked_down=blocked_down)
    h = synth.hidden(wl, 11)
    got, want, tr, gm = st.teal_step(h, 4096, kv_sparse, inject=True)
    assert rel_l2(got, want) <= TOL["bf16"]
    for k, n in enumerate(st.mask_sizes):
        assert abs(gm[0][k].mean() - 0.5) < 0.01, k


@pytest.mark.parametrize("blocked_down", [False, True])
@pytest.mark.parametrize("t_down", [1e30, -1.0])
def test_tiny_fp32_teal_step_down_input_all_dropped_or_all_kept(t_down, blocked_down):
    # the step decides the down projection's mask in the SwiGLU epilogue and
    # streams the kept rows (of w_down_t, or of the column blocks w_down_b):
    # with every down input dropped the MLP adds nothing, with t < 0 it reads
    # every row
    wl = synth.TINY
    st = TealStack(wl, 1, 1000, 300, blocked_down=blocked_down)
    h = synth.hidden(wl, 7).astype(np.float64)
    ts = st.thresholds(h, 1000, False, 0.5)
    ts = [(t[0], t[1], t[2], t_down) for t in ts]
    for k in range(4):
        st.layers[0].teal_t[k] = ts[0][k]
    hd = to_dev(h)
    sd.sd_decode_step(st.dims, st.layers, 1000, hd, sd.SD_PROJ_TEAL, st.ws)
    torch.cuda.synchronize()
    tr = []
    want = oteal.teal_step(st.olayers, h, 1000, ts, kv_sparse=False, trace=tr, **st.odims)
    assert rel_l2(to_host(hd), want) <= TOL["f32"]
    raw = st.teal_keep[0][1].cpu().numpy().astype(bool)
    down = raw[sum(st.mask_sizes[:3]):]
    assert down.size == wl.d_ff
    assert (not down.any()) if t_down > 0 else down.all()
    for k in range(4):
        cut = np.cumsum((0,) + st.mask_sizes)
        assert np.array_equal(raw[cut[k]:cut[k + 1]], tr[0]["masks"][k]), k


@pytest.mark.parametrize("d_in,d_out", [(32768, 4096), (32768, 8192), (4096, 8192), (4096, 8000),
                                        (6144, 1000)])
@pytest.mark.parametrize("norm", [False, True])
def test_teal_gemv_widest_inputs_and_ragged_last_block(d_in, d_out, norm):
    # the widest input the library accepts (32768 channels over 16 slices of
    # 2048), and outputs whose last 128-column block is partly padding
    # dims whose widths cover these sizes (the workspace is sized from them)
    wl = dataclasses.replace(synth.L8B_DENSE_8K, name="teal-widest", wid=7, d_model=8192,
                             n_q_heads=64, d_ff=32768)
    g = Gemv(wl, d_in, d_out, seed=d_in + d_out + 1)
    x = np.random.default_rng(d_out).standard_normal(d_in).astype(np.float32)
    xh = g.xhat(x, norm)
    t = midpoint_threshold(xh, 0.5)
    y, _, idx = g.run(x, t, norm)
    want, mask, widx = oteal.teal_linear(g.wt.T, xh, t)
    assert np.array_equal(idx, widx)
    assert rel_l2(y, want) <= TOL["bf16"]
