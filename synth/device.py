"""Device-side versions of the synthetic recipes (torch RNG on the GPU), for
stacks too large to draw on the host: 32 layers of 8B-class bf16 weights plus
caches of up to 128K rows.  Same distributions as synth; different random
streams (torch's Philox generator), seeded per (workload, layer, tensor)."""

from __future__ import annotations

import torch

from . import (T_DOWN, T_GATE, T_K, T_KSCALE, T_O, T_QKV, T_QWIN, T_UP, T_V, T_VSCALE, T_CAL,
               T_PLANT,
               T_H, Workload)


def _gen(wl: Workload, layer: int, tensor: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((wl.wid * 1000 + layer) * 100 + tensor) * 7919 + 17)
    return g


def _dt(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def normal(shape, std, wl, layer, tensor, device, dtype=None):
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=_gen(wl, layer, tensor, device))
    return t.to(dtype or _dt(wl))


def layer_weights(wl: Workload, layer: int, device) -> dict:
    d, f = wl.d_model, wl.d_ff
    hd = wl.n_q_heads * wl.head_dim
    return dict(
        attn_norm=torch.ones(d, device=device),
        w_qkv=normal((wl.qkv_out, d), 0.02, wl, layer, T_QKV, device),
        w_o=normal((d, hd), 0.02, wl, layer, T_O, device),
        mlp_norm=torch.ones(d, device=device),
        w_gate=normal((f, d), 0.02, wl, layer, T_GATE, device),
        w_up=normal((f, d), 0.02, wl, layer, T_UP, device),
        w_down_t=normal((f, d), 0.02, wl, layer, T_DOWN, device),
    )


def kv_cache(wl: Workload, layer: int, n: int, cap: int, device):
    """K, V [h_kv, cap, d_h]; rows >= n are zero; LogNormal(0, 0.5) channel scales."""
    out = []
    for tid, sid in ((T_K, T_KSCALE), (T_V, T_VSCALE)):
        x = torch.zeros(wl.n_kv_heads, cap, wl.head_dim, dtype=_dt(wl), device=device)
        z = torch.empty(wl.n_kv_heads, n, wl.head_dim, dtype=torch.float32, device=device)
        z.normal_(0.0, 1.0, generator=_gen(wl, layer, tid, device))
        if wl.channel_scale:
            s = torch.empty(wl.n_kv_heads, 1, wl.head_dim, dtype=torch.float32, device=device)
            s.log_normal_(0.0, 0.5, generator=_gen(wl, layer, sid, device))
            z.mul_(s)
        x[:, :n] = z.to(x.dtype)
        out.append(x)
    return out[0], out[1]


def window_queries(wl: Workload, layer: int, device):
    return normal((wl.n_q_heads, wl.window, wl.head_dim), 1.0, wl, layer, T_QWIN, device,
                  torch.float32)


def calibration_states(wl: Workload, layer: int, n_states: int, device):
    return normal((n_states, wl.d_model), 1.0, wl, layer, T_CAL, device, torch.float32)


def hidden(wl: Workload, draw: int, device):
    return normal((wl.d_model,), 1.0, wl, 1000 + draw, T_H, device, torch.float32)


def plant_keys(wl: Workload, layer: int, k, n: int, q_win, n_planted: int):
    """Device version of synth.plant_keys: n_planted positions drawn without
    replacement from [n_sink, n - window), shared by the KV heads; at each,
    head kv's key is 4 sqrt(d_h) times the unit vector of the sum of its query
    group's window queries.  Writes k in place; returns the sorted positions."""
    lo, hi = wl.n_sink, n - wl.window
    g = torch.Generator(device="cpu")
    g.manual_seed(((wl.wid * 1000 + layer) * 100 + T_PLANT) * 7919 + 17)
    pos = (torch.randperm(hi - lo, generator=g)[:n_planted] + lo).sort().values
    grp = wl.n_q_heads // wl.n_kv_heads
    s = q_win.double().reshape(wl.n_kv_heads, grp * wl.window, wl.head_dim).sum(dim=1)
    key = (4.0 * wl.head_dim ** 0.5) * s / s.norm(dim=1, keepdim=True)
    k[:, pos.to(k.device)] = key.to(k.dtype)[:, None, :]
    return pos


def teal_blocked(w, block: int = 128):
    """W [d_out, d_in] (nn.Linear order) in the column-block layout of the
    TEAL projections: [ceil(d_out / block)][d_in][block], columns past d_out
    zero.  A relayout only."""
    d_out, d_in = w.shape
    nblk = (d_out + block - 1) // block
    wt = torch.zeros(nblk * block, d_in, dtype=w.dtype, device=w.device)
    wt[:d_out] = w
    return wt.view(nblk, block, d_in).transpose(1, 2).contiguous()


def mma_tiles(w):
    """W [rows, d_in] (nn.Linear order) in the tile layout of the batched
    matrix-core projections: tiles of 16 rows by steps of 32 input channels,
    step-major, each (tile, step) in the A-operand lane order of the matrix
    core (lane l: row l % 16, channels 8 (l // 16) .. + 7 of the step),
    padding zero.  A relayout only."""
    rows, d_in = w.shape
    rp, kp = (rows + 15) // 16 * 16, (d_in + 31) // 32 * 32
    wp = torch.zeros(rp, kp, dtype=w.dtype, device=w.device)
    wp[:rows, :d_in] = w
    # [tile, r, step, q, e] -> [step, tile, q, r, e]: lane = r + 16 q
    return wp.view(rp // 16, 16, kp // 32, 4, 8).permute(2, 0, 3, 1, 4).contiguous()
