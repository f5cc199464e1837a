"""Stacked-layer parity at 8192 context on all 32 layers of the benchmark's
8B-class bf16 stack (built by bench.py's own Stack class, so weights, caches,
thresholds and launch configuration are the timed ones), in the composed mode
(KV keep 10% after the one-time selection, CATS sparsity 0.5) and in dense
mode.  The step runs through the C ABI one layer per call, and every layer's
output is checked against the float64 oracle run from the GPU's own input to
that layer, with the GPU's channel mask injected into the oracle (a channel
next to the threshold may flip between float32 paths; the flips are bounded
separately).  "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
Decoding", §4.1 (32-layer Llama-3.1-8B setting)."""

import ctypes
import types

import numpy as np
import pytest
import torch

from oracle import step as ostep

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import TOL, rel_l2, to_host  # noqa: E402

N = 8192


@pytest.fixture(scope="module")
def stack():
    import bench
    args = types.SimpleNamespace(contexts=str(N), layers=32, warmup=0, steps=2, blocks=1,
                                 block_steps=1)
    b = bench.Stack(args)
    _, k_keep = b.select(N)
    yield b, k_keep
    del b
    torch.cuda.empty_cache()


def _one_layer(b, li):
    return (sd.sd_layer * 1).from_address(ctypes.addressof(b.layers[li]))


def _oracle_layer(b, li):
    W = {k: to_host(v) for k, v in b.W[li].items() if k != "w_down_b"}
    L = b.layers[li]
    n, ns = L.n_full, L.n_sel
    return ostep.Layer(W["attn_norm"], W["w_qkv"], W["w_o"], W["mlp_norm"], W["w_gate"],
                       W["w_up"], W["w_down_t"], L.cats_threshold,
                       to_host(b.K[li][:, :n + 1]), to_host(b.V[li][:, :n + 1]), n,
                       to_host(b.KS[li][:, :ns + 1]), to_host(b.VS[li][:, :ns + 1]), ns)


@pytest.mark.parametrize("mode", ["both", "dense"])
def test_every_layer_matches_oracle(stack, mode):
    b, k_keep = stack
    wl = b.wl
    odims = dict(n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                 kv_dtype="bf16", eps=1e-5, theta=500000.0)
    flags = b.mode_flags(mode)
    kv_sparse = bool(flags & sd.SD_KV_SPARSE)
    mlp_sparse = bool(flags & sd.SD_MLP_SPARSE)
    b.reset(N, k_keep)
    errs = []
    for li in range(b.L):
        h_in = to_host(b.hidden).astype(np.float64)
        ol = _oracle_layer(b, li)
        sd.sd_decode_step(b.dims, _one_layer(b, li), N, b.hidden, flags, b.ws)
        torch.cuda.synchronize()
        got = to_host(b.hidden)
        gmask = b.MASK[li].cpu().numpy().astype(bool)
        if not mlp_sparse:
            assert gmask.all(), li
        tr = []
        want = ostep.decode_layer(ol, h_in, N, kv_sparse=kv_sparse, mlp_sparse=mlp_sparse,
                                  mask_override=gmask if mlp_sparse else None, trace=tr,
                                  **odims)
        err = rel_l2(got, want)
        errs.append(err)
        assert err <= TOL["bf16"], (mode, li, err)
        if mlp_sparse:
            own = tr[0]["act"].astype(np.float32)
            flips = int(np.sum((np.abs(own) > np.float32(ol.threshold)) != gmask))
            assert flips <= 0.002 * wl.d_ff, (li, flips)
            assert abs(gmask.mean() - 0.5) < 0.05, (li, gmask.mean())
        L = b.layers[li]
        assert L.n_full == N + 1 and L.n_sel == k_keep + 1
        krow = to_host(b.K[li][:, N])
        assert rel_l2(krow, ol.k_full[:, N]) <= TOL["bf16"]
        assert np.array_equal(to_host(b.KS[li][:, k_keep]), krow)
    print(f"{mode}: worst layer rel L2 {max(errs):.2e} (layer {int(np.argmax(errs))})")
