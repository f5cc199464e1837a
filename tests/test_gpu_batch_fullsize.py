"""GPU parity of the batched step ("Where Activation Sparsity and KV-Cache
Sparsity Cross in LLM Decoding", §3.3 "Dispatch and batching", §4.4
"Batching") at the size bench.py times it: 8 sequences at context 8192 on the
32-layer 8B-class bf16 stack, each with its own caches and one-time selection,
built by bench.py's own Stack and batch_caches, on the matrix cores (tile
weights packed by the library) and on the vector ALUs.

The oracle cannot run 32 layers for 8 sequences, so the step runs through the
C ABI one layer per call (each layer's kernels are launched exactly as in a
32-layer call) and sampled layers are checked against the float64 oracle from
the GPU's own input to that layer, every sequence.  At every one of the 32
layers, from a shared input, the two paths must agree with each other,
including the CATS union masks."""

import ctypes
import types

import numpy as np
import pytest
import torch

from oracle import step as ostep

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import DEV, TOL, rel_l2, to_host  # noqa: E402

N = 8192
B = 8
SAMPLED = (0, 31)


@pytest.fixture(scope="module")
def batch_stack():
    import bench
    args = types.SimpleNamespace(contexts=str(N), layers=32, warmup=0, steps=2, blocks=1,
                                 block_steps=1)
    b = bench.Stack(args)
    b.enable_tiles()
    caches = bench.batch_caches(b, N, B, grow=8)
    yield b, caches
    del caches
    b.disable_tiles()
    del b
    torch.cuda.empty_cache()


def _one_layer(b, li):
    return (sd.sd_layer * 1).from_address(ctypes.addressof(b.layers[li]))


def _oracle_layer(b, caches, li, bb):
    keep, kv, k_keep, _ = caches
    W = {k: to_host(v) for k, v in b.W[li].items() if k != "w_down_b"}
    k, v, ks, vs = keep[bb * b.L + li]
    return ostep.Layer(W["attn_norm"], W["w_qkv"], W["w_o"], W["mlp_norm"], W["w_gate"],
                       W["w_up"], W["w_down_t"], b.layers[li].cats_threshold,
                       to_host(k[:, :N + 1]), to_host(v[:, :N + 1]), N,
                       to_host(ks[:, :k_keep + 1]), to_host(vs[:, :k_keep + 1]), k_keep)


def _run(b, caches, flags, check=()):
    """One batched step through all layers, one layer per call, from context N;
    returns the final hidden states, the union mask of each layer, and the
    relative L2 errors of the checked layers against the oracle."""
    keep, kv, k_keep, h0 = caches
    L = b.L
    per = [(sd.sd_seq_kv * B)(*[kv[bb * L + li] for bb in range(B)]) for li in range(L)]
    hid = h0.clone()
    ws = torch.empty(sd.sd_batch_workspace_bytes(b.dims, B), dtype=torch.uint8, device=DEV)
    wl = b.wl
    odims = dict(n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                 kv_dtype="bf16", eps=1e-5, theta=500000.0)
    kv_sparse = bool(flags & sd.SD_KV_SPARSE)
    masks, errs = [], []
    for li in range(L):
        if li in check:
            h_in = to_host(hid).astype(np.float64)
            ol = [_oracle_layer(b, caches, li, bb) for bb in range(B)]
        sd.sd_decode_step_batch(b.dims, _one_layer(b, li), per[li], [N] * B, hid, flags, ws)
        torch.cuda.synchronize()
        masks.append(b.MASK[li].cpu().numpy().astype(bool))
        if li in check:
            got = to_host(hid)
            for bb in range(B):
                want = ostep.decode_layer(ol[bb], h_in[bb], N, kv_sparse=kv_sparse,
                                          mlp_sparse=False, **odims)
                errs.append((li, bb, rel_l2(got[bb], want)))
    for li in range(L):  # each call advanced its layer's counts by one row
        assert per[li][0].n_full == N + 1 and per[li][0].n_sel == k_keep + 1
    return to_host(hid), masks, errs


@pytest.mark.parametrize("matrix_cores", [True, False])
def test_batch_of_8_at_8k_sampled_layers_match_oracle(batch_stack, matrix_cores):
    b, caches = batch_stack
    flags = sd.SD_KV_SPARSE | (sd.SD_MATRIX_CORES if matrix_cores else 0)
    _, _, errs = _run(b, caches, flags, check=SAMPLED)
    assert len(errs) == len(SAMPLED) * B
    for li, bb, e in errs:
        assert e <= TOL["bf16"], (li, bb, e)


def _run_pair(b, caches, flags):
    """Both paths through all layers from the same input at every layer (the
    vector path's output feeds the next layer): per layer and sequence the
    relative L2 difference of the two outputs, and the union masks."""
    keep, kv, k_keep, h0 = caches
    L = b.L
    hid = h0.clone()
    ws = torch.empty(sd.sd_batch_workspace_bytes(b.dims, B), dtype=torch.uint8, device=DEV)
    diffs, masks = [], []
    for li in range(L):
        outs, ms = [], []
        for extra in (sd.SD_MATRIX_CORES, 0):
            per = (sd.sd_seq_kv * B)(*[kv[bb * L + li] for bb in range(B)])
            h = hid.clone()
            sd.sd_decode_step_batch(b.dims, _one_layer(b, li), per, [N] * B, h, flags | extra, ws)
            torch.cuda.synchronize()
            outs.append(to_host(h))
            ms.append(b.MASK[li].cpu().numpy().astype(bool))
        diffs.append([rel_l2(outs[0][bb], outs[1][bb]) for bb in range(B)])
        masks.append(ms)
        hid = torch.from_numpy(outs[1]).to(DEV)
    return np.array(diffs), masks


def test_batch_paths_agree_over_32_layers_with_cats(batch_stack):
    # KV 10% + CATS 0.5 through all 32 layers on both paths, each layer from
    # the same input.  The paths add in different orders, so an appended K or
    # V row can round to a different bf16 value and a gate value within
    # rounding of the threshold can be kept by one path only; run freely, a
    # flip in an early layer moves every later layer's input, so each layer
    # is compared from a shared input instead: outputs at the per-layer bf16
    # tolerance, union masks channel for channel to 99.9%
    b, caches = batch_stack
    both = sd.SD_KV_SPARSE | sd.SD_MLP_SPARSE
    diffs, masks = _run_pair(b, caches, both)
    assert diffs.shape == (b.L, B)
    assert diffs.max() <= TOL["bf16"], (np.unravel_index(diffs.argmax(), diffs.shape), diffs.max())
    for li, (m_mc, m_vec) in enumerate(masks):
        agree = float((m_mc == m_vec).mean())
        assert agree >= 0.999, (li, agree)
        # masks near 50% sparsity: the union of 8 keeps nearly every channel
        assert m_mc.mean() > 0.95, li
