"""GPU parity of sd_sparse_mlp (CATS gate, |a| > t mask, gathered up/down) and
sd_cats_calibrate against the float64 oracle."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import cats as ocats, step as ostep

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import (DEV, TOL, dims_for, midpoint_threshold, rel_l2, to_dev, to_host,  # noqa
                         workspace)


class Mlp:
    def __init__(self, wl, layer=0, weights=None):
        self.wl = wl
        self.dims = dims_for(wl)
        self.W = weights or synth.layer_weights(wl, layer)
        self.wg = to_dev(self.W["w_gate"], wl.dtype)
        self.wu = to_dev(self.W["w_up"], wl.dtype)
        self.wd = to_dev(self.W["w_down_t"], wl.dtype)
        self.norm = to_dev(self.W["mlp_norm"])
        self.y = torch.empty(wl.d_model, device=DEV)
        self.act = torch.empty(wl.d_ff, device=DEV)
        self.idx = torch.empty(wl.d_ff, dtype=torch.int32, device=DEV)
        self.n_kept = torch.empty(1, dtype=torch.int32, device=DEV)
        self.ws = workspace(self.dims)

    def run(self, x, t, norm=True, act_in=None):
        flags = 0
        if act_in is not None:
            self.act.copy_(torch.from_numpy(np.ascontiguousarray(act_in, np.float32)))
            flags = sd.SD_GATE_IN
        sd.sd_sparse_mlp(self.dims, to_dev(x), self.norm if norm else None, self.wg, self.wu,
                         self.wd, t, self.y, self.act, self.idx, self.n_kept, flags, self.ws)
        torch.cuda.synchronize()
        nk = int(self.n_kept.item())
        return to_host(self.y), to_host(self.act), self.idx.cpu().numpy()[:nk]

    def oracle(self, x, t, norm=True):
        xh = ostep.rmsnorm(x, self.W["mlp_norm"], 1e-5) if norm else np.asarray(x, np.float64)
        return ocats.cats_mlp(xh, self.W["w_gate"], self.W["w_up"], self.W["w_down_t"], t)


def test_tiny_dense_and_threshold_zero():
    m = Mlp(synth.TINY)
    x = synth.hidden(synth.TINY)
    for t in (-1.0, 0.0):
        y, act, idx = m.run(x, t)
        wy, wa, wmask, widx = m.oracle(x, t)
        assert rel_l2(act, wa) <= TOL["f32"]
        assert rel_l2(y, wy) <= TOL["f32"]
        assert np.array_equal(idx, widx) and idx.size == synth.TINY.d_ff


@pytest.mark.parametrize("sparsity", [0.3, 0.5, 0.7, 0.95])
def test_tiny_cats_matches_oracle(sparsity):
    wl = synth.TINY
    m = Mlp(wl)
    x = synth.hidden(wl, 1)
    _, a, _, _ = m.oracle(x, -1.0)
    t = midpoint_threshold(a, sparsity)
    y, act, idx = m.run(x, t)
    wy, wa, wmask, widx = m.oracle(x, t)
    assert rel_l2(act, wa) <= TOL["f32"]
    assert np.array_equal(idx, widx)
    assert idx.size == wl.d_ff - int(np.floor(sparsity * wl.d_ff + 0.5))
    assert rel_l2(y, wy) <= TOL["f32"]


def test_mask_bit_exact_on_oracle_activations_with_ties():
    # SD_GATE_IN: both sides decide |a| > t on the same float32 activations,
    # including entries exactly at +-t (dropped) and one ulp either side
    wl = synth.TINY
    m = Mlp(wl)
    x = synth.hidden(wl, 2)
    _, a, _, _ = m.oracle(x, -1.0)
    a32 = a.astype(np.float32)
    t = np.float32(np.median(np.abs(a32)))
    a32[:8] = [t, -t, np.nextafter(t, np.float32(1)), -np.nextafter(t, np.float32(1)),
               np.nextafter(t, np.float32(0)), 0.0, -0.0, 2 * t]
    y, act, idx = m.run(x, float(t), act_in=a32)
    wmask = ocats.cats_mask(a32, float(t))
    assert np.array_equal(idx, ocats.kept_indices(wmask))
    assert idx[:3].tolist() == [2, 3, 7]
    xh = ostep.rmsnorm(x, m.W["mlp_norm"], 1e-5)
    wy = ocats.mlp_masked(xh, m.W["w_gate"], m.W["w_up"], m.W["w_down_t"], wmask, act=a32)
    assert rel_l2(y, wy) <= TOL["f32"]


def test_no_norm_input_path():
    wl = synth.TINY
    m = Mlp(wl)
    x = synth.hidden(wl, 3) * 0.3
    y, act, idx = m.run(x, -1.0, norm=False)
    wy, wa, _, _ = m.oracle(x, -1.0, norm=False)
    assert rel_l2(y, wy) <= TOL["f32"] and rel_l2(act, wa) <= TOL["f32"]


@pytest.fixture(scope="module")
def mlp8b():
    return Mlp(synth.L8B_CATS_4K)


@pytest.mark.parametrize("sparsity", [0.0, 0.5, 0.7])
def test_8b_cats_matches_oracle(mlp8b, sparsity):
    # the CATS workload's layer: bf16 weights, d 4096, FFN 14336
    wl = synth.L8B_CATS_4K
    x = synth.hidden(wl, 0)
    _, a, _, _ = mlp8b.oracle(x, -1.0)
    t = midpoint_threshold(a, sparsity)
    y, act, idx = mlp8b.run(x, t)
    wy, wa, wmask, widx = mlp8b.oracle(x, t)
    assert rel_l2(act, wa) <= TOL["bf16"]
    assert np.array_equal(idx, widx)
    assert rel_l2(y, wy) <= TOL["bf16"]
    assert rel_l2(y, wy) <= 1e-5  # float32 accumulation over exact bf16 weights


def test_8b_deterministic(mlp8b):
    wl = synth.L8B_CATS_4K
    x = synth.hidden(wl, 4)
    a = mlp8b.run(x, 0.05)
    b = mlp8b.run(x, 0.05)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))


@pytest.mark.parametrize("sparsity", [0.0, 0.5, 0.7, 1.0])
def test_calibration_matches_oracle(sparsity):
    # threshold = k-th smallest |SiLU(gate)| over calibration states
    wl = dataclasses.replace(synth.L8B_CATS_4K, d_ff=2048)
    W = synth.layer_weights(wl, 0)
    states = synth.calibration_states(wl, 0, 64)
    dims = dims_for(wl)
    ws = torch.empty(sd.sd_calibrate_workspace_bytes(dims, 64), dtype=torch.uint8, device=DEV)
    thr = torch.empty(1, device=DEV)
    sd.sd_cats_calibrate(dims, to_dev(states), 64, to_dev(W["mlp_norm"]),
                         to_dev(W["w_gate"], "bf16"), sparsity, thr, ws)
    torch.cuda.synchronize()
    got = float(thr.item())
    xs = [ostep.rmsnorm(s, W["mlp_norm"], 1e-5) for s in states]
    vals = np.abs(np.stack([ocats.gate_act(x, W["w_gate"]) for x in xs]).astype(np.float32))
    want = ocats.calibrate_threshold(vals, sparsity)
    if want < 0:
        assert got == -1.0
    else:
        assert abs(got - want) <= 1e-5 * abs(want)


def _mlp_weights(wl):
    """The three MLP matrices of `wl` (seeded as synth.layer_weights draws them)."""
    f, d = wl.d_ff, wl.d_model

    def w(tid):
        return synth._cast(synth.rng(wl.wid, 0, tid).standard_normal((f, d), dtype=np.float32)
                           * 0.02, wl.dtype)

    return dict(mlp_norm=np.ones(d, np.float32), w_gate=w(synth.T_GATE), w_up=w(synth.T_UP),
                w_down_t=w(synth.T_DOWN))


@pytest.mark.parametrize("sparsity", [0.0, 0.5])
def test_max_size_cats_matches_oracle(sparsity):
    # the largest sizes the library accepts: d_model 8192 (the widest GEMV
    # input) and d_ff 32768 (512 down slices of at most 64 kept channels;
    # keeping every channel fills every slice exactly)
    wl = dataclasses.replace(synth.L8B_CATS_4K, name="max-width-cats", wid=5, d_model=8192,
                             n_q_heads=64, d_ff=32768)
    m = Mlp(wl, weights=_mlp_weights(wl))
    x = synth.hidden(wl, 2)
    _, a, _, _ = m.oracle(x, -1.0)
    t = midpoint_threshold(a, sparsity) if sparsity > 0 else -1.0
    y, act, idx = m.run(x, t)
    wy, wa, wmask, widx = m.oracle(x, t)
    assert rel_l2(act, wa) <= TOL["bf16"]
    assert np.array_equal(idx, widx)
    assert idx.size == (wl.d_ff if sparsity == 0 else wl.d_ff // 2)
    assert rel_l2(y, wy) <= TOL["bf16"]
