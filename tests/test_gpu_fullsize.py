"""GPU parity at the full size of the composed workload that bench.py times:
32 stacked 8B-class bf16 layers at context 131072, KV keep 10% (one-time
selection), CATS thresholds calibrated for sparsity 0.5 -- built by bench.py's
own Stack class, so the launch configuration is the timed one.

The oracle cannot run the whole stack, so the step runs through the C ABI one
layer per call (every layer's kernels are launched exactly as in a 32-layer
call), and sampled layers are checked one by one against the float64 oracle
from the GPU's own input to that layer.  The selection of a sampled layer is
checked at 131072 context, and the whole stack for run-to-run determinism.
The TEAL + KV step (all seven projections sparse, thresholds calibrated by
the benchmark's own harness) is checked the same way."""

import ctypes
import math
import types

import numpy as np
import pytest
import torch

from oracle import selection as osel, step as ostep, teal as oteal

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import TOL, rel_l2, to_host  # noqa: E402

N = 131072
SAMPLED = (0, 31)


@pytest.fixture(scope="module")
def stack():
    import bench
    args = types.SimpleNamespace(contexts=str(N), layers=32, warmup=0, steps=2, blocks=1,
                                 block_steps=1)
    b = bench.Stack(args)
    b.enable_teal()
    secs, k_keep = b.select(N)
    yield b, k_keep
    del b
    torch.cuda.empty_cache()


def _one_layer(b, li):
    """ctypes view of layers[li] as a 1-layer array (n_full / n_sel advance in place)."""
    return (sd.sd_layer * 1).from_address(ctypes.addressof(b.layers[li]))


def _oracle_layer(b, li, k_keep):
    W = {k: to_host(v) for k, v in b.W[li].items() if k != "w_down_b"}
    L = b.layers[li]
    n, ns = L.n_full, L.n_sel
    k = to_host(b.K[li][:, :n + 1])
    v = to_host(b.V[li][:, :n + 1])
    ks = to_host(b.KS[li][:, :ns + 1])
    vs = to_host(b.VS[li][:, :ns + 1])
    return ostep.Layer(W["attn_norm"], W["w_qkv"], W["w_o"], W["mlp_norm"], W["w_gate"],
                       W["w_up"], W["w_down_t"], L.cats_threshold, k, v, n, ks, vs, ns)


def test_composed_step_sampled_layers_match_oracle(stack):
    b, k_keep = stack
    wl = b.wl
    odims = dict(n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                 kv_dtype="bf16", eps=1e-5, theta=500000.0)
    b.reset(N, k_keep)
    mode = sd.SD_KV_SPARSE | sd.SD_MLP_SPARSE
    for li in range(b.L):
        if li in SAMPLED:
            h_in = to_host(b.hidden).astype(np.float64)
            ol = _oracle_layer(b, li, k_keep)
        sd.sd_decode_step(b.dims, _one_layer(b, li), N, b.hidden, mode, b.ws)
        if li not in SAMPLED:
            continue
        torch.cuda.synchronize()
        got = to_host(b.hidden)
        gmask = b.MASK[li].cpu().numpy().astype(bool)
        tr = []
        # P-C: the oracle with the GPU's channel mask injected
        want = ostep.decode_layer(ol, h_in, N, kv_sparse=True, mlp_sparse=True,
                                  mask_override=gmask, trace=tr, **odims)
        err = rel_l2(got, want)
        assert err <= TOL["bf16"], (li, err)
        # P-D (informational bound): the oracle's own mask differs only near t
        own = tr[0]["act"].astype(np.float32)
        flips = int(np.sum((np.abs(own) > np.float32(ol.threshold)) != gmask))
        assert flips <= 0.002 * wl.d_ff, (li, flips)
        # the appended row landed in both buffers, rounded like the oracle's
        L = b.layers[li]
        krow = to_host(b.K[li][:, L.n_full - 1])
        assert rel_l2(krow, ol.k_full[:, L.n_full - 1]) <= TOL["bf16"]
        assert np.array_equal(to_host(b.KS[li][:, L.n_sel - 1]), krow)


def test_selection_at_full_context(stack):
    b, k_keep = stack
    wl = b.wl
    li = SAMPLED[0]
    k = to_host(b.K[li][:, :N])
    qw = to_host(b.QW[li])
    sd.sd_select_kv(b.dims, b.K[li], b.V[li], b.cap_full, N, b.QW[li], wl.window, wl.n_sink,
                    k_keep, b.scores, b.idx, b.KS[li], b.VS[li], b.cap_sel, 0, b.ws)
    torch.cuda.synchronize()
    got_s = to_host(b.scores[:, :N])
    want_s = osel.window_scores(qw, k, N, 1 / math.sqrt(wl.head_dim))
    assert rel_l2(got_s, want_s) <= 1e-5
    np.testing.assert_allclose(got_s.sum(1), (wl.n_q_heads // wl.n_kv_heads) * wl.window,
                               rtol=1e-4)
    # the ranking of the GPU's float32 scores equals the oracle's ranking of them
    got_idx = b.idx[:wl.n_kv_heads * k_keep].view(wl.n_kv_heads, k_keep).cpu().numpy()
    want_idx = osel.select_indices(got_s.astype(np.float32), N, wl.window, wl.n_sink, k_keep)
    assert np.array_equal(got_idx, want_idx)
    ks = b.KS[li][:, :k_keep].contiguous().view(torch.int16).cpu().numpy()
    kf = b.K[li].view(torch.int16).cpu().numpy()
    assert np.array_equal(ks, np.stack([kf[h, want_idx[h]] for h in range(wl.n_kv_heads)]))


def test_whole_stack_is_deterministic(stack):
    b, k_keep = stack
    outs = []
    for _ in range(2):
        b.reset(N, k_keep)
        b.run_steps(N, sd.SD_KV_SPARSE | sd.SD_MLP_SPARSE, 2)
        torch.cuda.synchronize()
        outs.append(b.hidden.cpu().numpy().copy())
    assert np.array_equal(outs[0], outs[1])
    assert np.all(np.isfinite(outs[0]))


def test_teal_kv_step_sampled_layers_match_oracle(stack):
    b, k_keep = stack
    wl = b.wl
    odims = dict(n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                 kv_dtype="bf16", eps=1e-5, theta=500000.0)
    mode = sd.SD_KV_SPARSE | sd.SD_PROJ_TEAL
    b.teal_calibrate(N, k_keep, mode)
    cut = np.cumsum((0,) + tuple(b.teal_sizes))
    b.reset(N, k_keep)
    for li in range(b.L):
        if li in SAMPLED:
            h_in = to_host(b.hidden).astype(np.float64)
            ol = _oracle_layer(b, li, k_keep)
        sd.sd_decode_step(b.dims, _one_layer(b, li), N, b.hidden, mode, b.ws)
        if li not in SAMPLED:
            continue
        torch.cuda.synchronize()
        got = to_host(b.hidden)
        tm = b.TMASK[li].cpu().numpy().astype(bool)
        gm = [tm[cut[k]:cut[k + 1]] for k in range(4)]
        t = [float(b.layers[li].teal_t[k]) for k in range(4)]
        tr = []
        # the oracle with the GPU's four masks injected
        want = oteal.teal_layer(ol, h_in, N, t, kv_sparse=True, masks=gm, trace=tr, **odims)
        err = rel_l2(got, want)
        assert err <= TOL["bf16"], (li, err)
        # the GPU's masks against the oracle's own decisions on the oracle's
        # inputs: they differ only next to the threshold (informational bound)
        own = (tr[0]["x"], tr[0]["attn"], tr[0]["x2"], tr[0]["hmid"])
        for k in range(4):
            flips = int(np.sum(oteal.teal_mask(own[k].astype(np.float32), t[k]) != gm[k]))
            assert flips <= 0.005 * gm[k].size + 4, (li, k, flips)
            assert abs(gm[k].mean() - 0.5) < 0.1, (li, k, gm[k].mean())
