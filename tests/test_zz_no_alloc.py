"""sd_decode_step_noalloc (the decode step on the library's own per-GPU
scratch buffer, for callers that cannot allocate) against sd_decode_step with
a caller workspace, through the C ABI: two calls in a row on the same GPU, the
second with a smaller input, each compared element by element (relative L2
within the float32 tolerance, and the appended cache rows)."""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import DEV, TOL, dims_for, rel_l2, to_dev, to_host, workspace  # noqa: E402


class Twin:
    """Two identical copies of an n-row decode state over shared weights: one
    for each entry point."""

    def __init__(self, wl, n_layers, n, k_keep, threshold):
        self.dims = dims_for(wl)
        self.keep = []
        self.sets = []
        W = [synth.layer_weights(wl, li) for li in range(n_layers)]
        dW = [{k: to_dev(v, "f32" if "norm" in k else wl.dtype) for k, v in w.items()}
              for w in W]
        cap = n + 8
        for _ in range(2):
            layers = []
            for li in range(n_layers):
                k, v = synth.kv_cache(wl, li, n, cap)
                ks = np.zeros((wl.n_kv_heads, k_keep + 8, wl.head_dim), np.float32)
                vs = np.zeros_like(ks)
                ks[:, :k_keep] = k[:, :k_keep]  # any gathered rows serve the comparison
                vs[:, :k_keep] = v[:, :k_keep]
                t = [to_dev(a, wl.dtype) for a in (k, v, ks, vs)]
                mask = torch.zeros(wl.d_ff, dtype=torch.uint8, device=DEV)
                self.keep.append((t, mask))
                w = dW[li]
                layers.append(sd.sd_layer(
                    w["attn_norm"].data_ptr(), w["w_qkv"].data_ptr(), w["w_o"].data_ptr(),
                    w["mlp_norm"].data_ptr(), w["w_gate"].data_ptr(), w["w_up"].data_ptr(),
                    w["w_down_t"].data_ptr(), threshold, 0, t[0].data_ptr(), t[1].data_ptr(),
                    cap, n, t[2].data_ptr(), t[3].data_ptr(), k_keep + 8, k_keep,
                    mask.data_ptr()))
            self.sets.append((sd.sd_layer * n_layers)(*layers))
        self.keep.append(dW)
        self.n_layers = n_layers

    def caches(self, which):
        per = len(self.keep[:-1]) // 2
        return self.keep[which * per:(which + 1) * per]


def _compare(wl, n_layers, n, k_keep, threshold, mode, draw):
    tw = Twin(wl, n_layers, n, k_keep, threshold)
    h0 = synth.hidden(wl, draw)
    ha, hb = to_dev(h0), to_dev(h0)
    ws = workspace(tw.dims)
    sd.sd_decode_step(tw.dims, tw.sets[0], n, ha, mode, ws)
    sd.sd_decode_step_noalloc(tw.dims, tw.sets[1], n, hb, mode)
    torch.cuda.synchronize()
    got, want = to_host(hb), to_host(ha)
    assert np.all(np.isfinite(got))
    assert rel_l2(got, want) <= TOL["f32"], rel_l2(got, want)
    for (ta, ma), (tb, mb) in zip(tw.caches(0), tw.caches(1)):
        for a, b in zip(ta, tb):  # full caches and gathered buffers, appended rows included
            assert rel_l2(to_host(b), to_host(a)) <= TOL["f32"]
        assert torch.equal(ma, mb)
    for la, lb in zip(tw.sets[0], tw.sets[1]):
        assert (la.n_full, la.n_sel) == (lb.n_full, lb.n_sel) == (n + 1, k_keep + 1)


def test_noalloc_matches_workspace_step_twice_second_smaller():
    # first call: 8B-class bf16 layers, two of them, composed mode at 4096 rows
    wl = synth.L8B_DENSE_8K
    _compare(wl, 2, 4096, 512, 0.05, sd.SD_KV_SPARSE | sd.SD_MLP_SPARSE, 3)
    # second call, smaller: one tiny float32 layer at 300 rows, dense
    _compare(synth.TINY, 1, 300, 64, -1.0, 0, 4)


def test_noalloc_rejects_a_step_beyond_its_buffer():
    # the masked comparison path needs score rows for every allocated row:
    # 32 query heads x 2^20 rows x 4 bytes exceeds the 64 MiB buffer
    wl = synth.L8B_DENSE_8K
    dims = dims_for(wl)
    big = 1 << 20
    L = sd.sd_layer()
    L.cap_full = big
    layers = (sd.sd_layer * 1)(L)
    h = torch.zeros(wl.d_model, device=DEV)
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step_noalloc(dims, layers, 0, h, sd.SD_ATTN_MASKED)
    assert e.value.status == sd.SD_ENOSPC
    assert "scratch" in sd.sd_last_error()
