#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X.

Workload: 32 stacked 8B-class layers (d 4096, 32/8 heads, head_dim 128, FFN
14336, bf16 weights and caches) with independent N(0, 0.02^2) weights and
synthetic caches (K, V ~ N(0,1) times LogNormal(0, 0.5) channel scales), in
four modes: dense, KV (10% keep, one-time attention-scored selection), CATS
(thresholds for 50% gate sparsity from 256 Gaussian calibration states per
layer) and both, over contexts from 2K to 128K.  The headline is the
composed step ("both") at 131072.

A step is one call of sd_decode_step through all 32 layers (each layer
appends its key/value row, so the context grows by one per step).  Inputs are
resident in HBM before timing.

Timing follows "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
Decoding" (§4.1 "Timing and quality", §4.3): per cell a discarded warm-up
block, then `--blocks` blocks of `--block-steps` decode steps, HIP events on
the library's stream at every block boundary; a cell's time is the median
block (min and max beside it).  The headline `value` and `ms_per_step` come
from their own timed region: `--warmup` untimed steps, then exactly `--steps`
steps between a device synchronize and events on both sides.

value = algorithmic HBM bytes per step / time per step (GB/s, 1e9 bytes):
weights read (QKV, O, gate, kept up rows, kept down rows), cached K/V rows
read, and the appended rows written.

The last line on stdout is one compact JSON record; every other leg (single
layer cells, crossing, TEAL, CateKV, batched decode, attention baselines,
latency gate, per-kernel times) is printed on '#' lines before it and, with
--out, written in full to that file.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("decode-step µs and achieved HBM GB/s (% of peak) vs context length, "
          "dense/KV/CATS/both")
HBM_PEAK_GBS = 8000.0
HEAD_MODES = ("dense", "kv", "cats", "both")
# CateKV's benchmark setting: 40% of the KV heads adaptive (eta = 1 keeps all
# their entries), the others keep a budget of 2048
CATEKV_RATIO, CATEKV_ETA, CATEKV_BUDGET = 0.4, 1.0, 2048
# decode lengths over which the latency gate charges one-time selection
GATE_HORIZONS = (256, 1024, 4096, 16384)
LEGS = ("head", "sweep", "cells", "teal", "catekv", "batch", "baselines", "cpu")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of the headline cell")
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps before them")
    ap.add_argument("--blocks", type=int, default=5, help="timed blocks per sweep cell")
    ap.add_argument("--block-steps", type=int, default=50, help="decode steps per block")
    ap.add_argument("--contexts", type=str,
                    default="2048,8192,16384,24576,32768,49152,65536,131072")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--legs", type=str, default=",".join(LEGS))
    ap.add_argument("--modes", type=str, default=",".join(HEAD_MODES),
                    help="modes of the sweep (the crossing needs all four)")
    ap.add_argument("--teal-contexts", type=str, default="32768,131072")
    ap.add_argument("--teal-modes", type=str, default="teal,teal+kv")
    ap.add_argument("--catekv-contexts", type=str, default="32768,131072")
    ap.add_argument("--batches", type=str, default="4,8")
    ap.add_argument("--batch-contexts", type=str, default="8192,32768")
    ap.add_argument("--batch-modes", type=str, default=",".join(HEAD_MODES))
    ap.add_argument("--batch-paths", type=str, default="vector,matrix_cores",
                    help="batched projections on the vector ALUs and/or the matrix cores")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--out", type=str, default="")
    ap.add_argument("--pmc-copy-bytes", type=int, default=0,
                    help="start with three plain device copies of this many bytes (counter "
                         "calibration for rocprofv3 --pmc runs)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter CSVs of this script into "
                         "per-kernel HBM bytes (needs --pmc-copy-bytes of those runs)")
    ap.add_argument("--pmc-out", type=str, default=TRAFFIC_JSON)
    ap.add_argument("--trace-summary", type=str, metavar="KERNEL_TRACE_CSV",
                    help="no GPU: per-kernel durations from a rocprofv3 --kernel-trace CSV of "
                         "this script, as a markdown summary (--trace-out, --trace-title, "
                         "--trace-cmd)")
    ap.add_argument("--trace-out", type=str, default="")
    ap.add_argument("--trace-title", type=str, default="")
    ap.add_argument("--trace-cmd", type=str, default="")
    return ap.parse_args()


def note(tag, obj):
    """One '#' line of a leg's results (compact JSON)."""
    print(f"# {tag} {json.dumps(obj, separators=(',', ':'))}", flush=True)


def rnd(x, nd=4):
    if isinstance(x, float):
        return round(x, nd)
    if isinstance(x, dict):
        return {k: rnd(v, nd) for k, v in x.items()}
    if isinstance(x, (list, tuple)):
        return [rnd(v, nd) for v in x]
    return x


class Stack:
    """The 32-layer stack: weights, full caches, gathered buffers, window
    queries and CATS thresholds, all resident on the GPU."""

    def __init__(self, args):
        import torch

        import kv_cache_activation_amd as sd
        import synth
        from synth import device as sdev

        self.torch, self.sd, self.synth = torch, sd, synth
        self.args = args
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()
        wl = synth.STACK32_128K
        self.wl = wl
        self.L = args.layers
        self.contexts = sorted(int(c) for c in args.contexts.split(","))
        n_max = max(self.contexts)
        # rows appended by the longest timed run of one cell
        self.grow = (1 + args.blocks) * args.block_steps + args.warmup + args.steps + 8
        self.cap_full = n_max + self.grow + 64
        self.cap_sel = int(math.floor(wl.keep_ratio * n_max)) + self.grow + 64
        self.dims = sd.make_dims(wl.d_model, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff,
                                 sd.SD_BF16, sd.SD_BF16)
        self.ws = torch.empty(sd.sd_workspace_bytes(self.dims, self.cap_full, wl.window),
                              dtype=torch.uint8, device=self.dev)
        self.W, self.K, self.V, self.KS, self.VS, self.QW, self.MASK = [], [], [], [], [], [], []
        for li in range(self.L):
            self.W.append(sdev.layer_weights(wl, li, self.dev))
            k, v = sdev.kv_cache(wl, li, n_max, self.cap_full, self.dev)
            self.K.append(k)
            self.V.append(v)
            self.KS.append(torch.zeros(wl.n_kv_heads, self.cap_sel, wl.head_dim,
                                       dtype=torch.bfloat16, device=self.dev))
            self.VS.append(torch.zeros_like(self.KS[-1]))
            self.QW.append(sdev.window_queries(wl, li, self.dev))
            self.MASK.append(torch.zeros(wl.d_ff, dtype=torch.uint8, device=self.dev))
        self.scores = torch.empty(wl.n_kv_heads, n_max, device=self.dev)
        self.idx = torch.empty(wl.n_kv_heads * n_max, dtype=torch.int32, device=self.dev)
        self.h0 = sdev.hidden(wl, 0, self.dev)
        self.hidden = self.h0.clone()
        self.thresholds = self.calibrate(range(self.L), 0.5)
        layers = []
        for li in range(self.L):
            W = self.W[li]
            layers.append(sd.sd_layer(
                W["attn_norm"].data_ptr(), W["w_qkv"].data_ptr(), W["w_o"].data_ptr(),
                W["mlp_norm"].data_ptr(), W["w_gate"].data_ptr(), W["w_up"].data_ptr(),
                W["w_down_t"].data_ptr(), self.thresholds[li], 0, self.K[li].data_ptr(),
                self.V[li].data_ptr(), self.cap_full, 0, self.KS[li].data_ptr(),
                self.VS[li].data_ptr(), self.cap_sel, 0, self.MASK[li].data_ptr()))
            # the down projection in column blocks of 128 outputs as well
            W["w_down_b"] = sdev.teal_blocked(W["w_down_t"].t())
            layers[-1].w_down_b = W["w_down_b"].data_ptr()
        self.layers = (sd.sd_layer * self.L)(*layers)
        self.ragged = False
        self.teal = False
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- set-up
    def calibrate(self, layers, sparsity, n_states=256):
        """CATS thresholds of the given layers (harness: 256 Gaussian states
        per layer through RMSNorm and the gate, percentile rule)."""
        torch, sd = self.torch, self.sd
        from synth import device as sdev
        ws = torch.empty(sd.sd_calibrate_workspace_bytes(self.dims, n_states), dtype=torch.uint8,
                         device=self.dev)
        layers = list(layers)
        thr = torch.empty(len(layers), device=self.dev)
        for i, li in enumerate(layers):
            states = sdev.calibration_states(self.wl, li, n_states, self.dev)
            sd.sd_cats_calibrate(self.dims, states, n_states, self.W[li]["mlp_norm"],
                                 self.W[li]["w_gate"], sparsity, thr[i:i + 1], ws)
        return thr.cpu().tolist()

    def enable_ragged(self):
        """CateKV: one gathered buffer per layer with a budget per KV head."""
        import ctypes
        torch, wl = self.torch, self.wl
        n_max = max(self.contexts)
        self.adaptive = self.synth.catekv_adaptive(wl, self.L, CATEKV_RATIO)
        self.cap_r = n_max + self.grow + 64
        self.KR, self.VR, self.RH = [], [], []
        for li in range(self.L):
            self.KR.append(torch.zeros(wl.n_kv_heads, self.cap_r, wl.head_dim,
                                       dtype=torch.bfloat16, device=self.dev))
            self.VR.append(torch.zeros_like(self.KR[-1]))
            self.RH.append((ctypes.c_int32 * wl.n_kv_heads)())
        self.ragged_keep = None
        self.ragged = True

    def disable_ragged(self):
        self.use_ragged(False)
        del self.KR, self.VR
        self.ragged = False
        self.torch.cuda.empty_cache()

    def enable_teal(self):
        """TEAL reads the projections in column blocks of 128 outputs,
        [ceil(d_out / 128)][d_in][128]."""
        from synth import device as sdev
        torch, wl = self.torch, self.wl
        self.WT, self.TMASK = [], []
        d, qd, ff = wl.d_model, wl.n_q_heads * wl.head_dim, wl.d_ff
        self.teal_sizes = (d, qd, d, ff)
        for li in range(self.L):
            W = self.W[li]
            wt = {k: sdev.teal_blocked(W[k]) for k in ("w_qkv", "w_o", "w_gate", "w_up")}
            self.WT.append(wt)
            self.TMASK.append(torch.zeros(sum(self.teal_sizes), dtype=torch.uint8,
                                          device=self.dev))
            L = self.layers[li]
            L.w_qkv_t, L.w_o_t = wt["w_qkv"].data_ptr(), wt["w_o"].data_ptr()
            L.w_gate_t, L.w_up_t = wt["w_gate"].data_ptr(), wt["w_up"].data_ptr()
            L.teal_masks_out = self.TMASK[li].data_ptr()
        self.teal = True

    def disable_teal(self):
        for L in self.layers:
            L.w_qkv_t = L.w_o_t = L.w_gate_t = L.w_up_t = None
            L.teal_masks_out = None
        del self.WT, self.TMASK
        self.teal = False
        self.torch.cuda.empty_cache()

    def enable_tiles(self):
        """The batched matrix-core path reads the five projections in 16-row x
        32-channel tiles, packed on the device by the library."""
        torch, sd = self.torch, self.sd
        self.TILES = []
        for li in range(self.L):
            W, L, t = self.W[li], self.layers[li], {}
            for f, w in (("w_qkv_m", W["w_qkv"]), ("w_o_m", W["w_o"]), ("w_gate_m", W["w_gate"]),
                         ("w_up_m", W["w_up"]), ("w_down_m", W["w_down_t"].t().contiguous())):
                t[f] = torch.empty(sd.sd_tile_bytes(*w.shape), dtype=torch.uint8, device=self.dev)
                sd.sd_pack_tiles(w, w.shape[0], w.shape[1], t[f])
                setattr(L, f, t[f].data_ptr())
            self.TILES.append(t)
        torch.cuda.synchronize()

    def disable_tiles(self):
        for L in self.layers:
            L.w_qkv_m = L.w_o_m = L.w_gate_m = L.w_up_m = L.w_down_m = None
        del self.TILES
        self.torch.cuda.empty_cache()

    # -------------------------------------------------------------- stepping
    def select(self, n):
        """One-time selection at context n for every layer; returns seconds."""
        torch, sd, wl = self.torch, self.sd, self.wl
        k_keep = int(math.floor(wl.keep_ratio * n))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for li in range(self.L):
            sd.sd_select_kv(self.dims, self.K[li], self.V[li], self.cap_full, n, self.QW[li],
                            wl.window, wl.n_sink, k_keep, self.scores, self.idx, self.KS[li],
                            self.VS[li], self.cap_sel, 0, self.ws)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, k_keep

    def catekv_budgets(self, n, li):
        return [min(n, int(math.floor(CATEKV_ETA * n))) if a else min(n, CATEKV_BUDGET)
                for a in self.adaptive[li]]

    def select_ragged(self, n):
        """One-time CateKV selection at context n for every layer (same scores
        and ranking as select(), one budget per KV head); returns seconds."""
        torch, sd, wl = self.torch, self.sd, self.wl
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        keep = []
        for li in range(self.L):
            kh = self.catekv_budgets(n, li)
            sd.sd_select_kv_ragged(self.dims, self.K[li], self.V[li], self.cap_full, n,
                                   self.QW[li], wl.window, wl.n_sink, kh, self.scores, self.idx,
                                   n, self.KR[li], self.VR[li], self.cap_r, 0, self.ws)
            keep.append(kh)
        torch.cuda.synchronize()
        self.ragged_keep = keep
        return time.perf_counter() - t0

    def use_ragged(self, on):
        """Point every layer at the CateKV buffers (on) or the uniform ones."""
        for li, L in enumerate(self.layers):
            if on:
                L.k_sel, L.v_sel = self.KR[li].data_ptr(), self.VR[li].data_ptr()
                L.cap_sel, L.n_sel_heads = self.cap_r, self.RH[li]
            else:
                L.k_sel, L.v_sel = self.KS[li].data_ptr(), self.VS[li].data_ptr()
                L.cap_sel, L.n_sel_heads = self.cap_sel, None

    def reset(self, n, k_keep, ragged=False):
        if self.ragged:
            self.use_ragged(ragged)
        for li, L in enumerate(self.layers):
            L.n_full = n
            L.n_sel = k_keep
            if ragged:
                for h, k in enumerate(self.ragged_keep[li]):
                    self.RH[li][h] = k
        self.hidden.copy_(self.h0)

    def run_steps(self, n, mode_flags, count):
        for i in range(count):
            self.sd.sd_decode_step(self.dims, self.layers, n + i, self.hidden, mode_flags, self.ws)

    def mode_flags(self, mode):
        sd = self.sd
        return {"dense": 0, "kv": sd.SD_KV_SPARSE, "cats": sd.SD_MLP_SPARSE,
                "both": sd.SD_KV_SPARSE | sd.SD_MLP_SPARSE, "teal": sd.SD_PROJ_TEAL,
                "teal+kv": sd.SD_PROJ_TEAL | sd.SD_KV_SPARSE, "catekv": sd.SD_KV_SPARSE,
                "catekv+cats": sd.SD_KV_SPARSE | sd.SD_MLP_SPARSE}[mode]

    # ----------------------------------------------------------------- bytes
    def step_bytes(self, n_read, n_kept_mean, layers=None):
        wl = self.wl
        d, dh = wl.d_model, wl.head_dim
        w = 2 * (d * wl.qkv_out + wl.n_q_heads * dh * d + d * wl.d_ff + 2 * d * n_kept_mean)
        row = 2 * wl.n_kv_heads * dh * 2
        return (layers or self.L) * (w + row * n_read + 2 * row)

    def teal_keep_fractions(self):
        """Per layer, the kept fraction of each of the four TEAL inputs in the
        last step (from the step's own mask output)."""
        cut = [0]
        for n in self.teal_sizes:
            cut.append(cut[-1] + n)
        out = []
        for m in self.TMASK:
            v = m.float()
            out.append([float(v[cut[k]:cut[k + 1]].mean()) for k in range(4)])
        return out

    def teal_step_bytes(self, n_read, fr):
        """Algorithmic bytes of a TEAL step: each projection's kept rows (mean
        kept fraction of its input over the layers) plus the cache rows."""
        wl = self.wl
        d, qd, ff = wl.d_model, wl.n_q_heads * wl.head_dim, wl.d_ff
        f = [sum(x[k] for x in fr) / len(fr) for k in range(4)]
        w = 2 * (d * wl.qkv_out * f[0] + qd * d * f[1] + 2 * d * ff * f[2] + ff * d * f[3])
        row = 2 * wl.n_kv_heads * wl.head_dim * 2
        return self.L * (w + row * n_read + 2 * row), f

    def teal_calibrate(self, n, k_keep, flags, target=0.5, iters=18, tol=0.01, refine=40):
        """TEAL thresholds (harness): per layer and input, the threshold at which
        the step keeps the target fraction of that input (one decode step per
        round, from the same state each time).  The page calibrates TEAL's
        magnitude thresholds offline to 50% keep; here the synthetic inputs'
        own magnitudes stand in for calibration data.  A bisection in log space
        moves every threshold at once; since an input's magnitudes depend on
        the thresholds before it (earlier layers, earlier inputs of its layer),
        a bracket can close on a target that later moves, so damped Newton
        steps in log t follow (slope of a half-normal's kept fraction at its
        median, about -0.43 per unit of log t; a threshold's step is halved
        whenever its error changes sign and grows back while it keeps its
        sign) until every input keeps within `tol` of the target."""
        lo = [[math.log(1e-6)] * 4 for _ in range(self.L)]
        hi = [[math.log(1e3)] * 4 for _ in range(self.L)]
        logt = [[0.0] * 4 for _ in range(self.L)]

        def fractions():
            for li, L in enumerate(self.layers):
                for k in range(4):
                    L.teal_t[k] = math.exp(logt[li][k])
            self.reset(n, k_keep)
            self.run_steps(n, flags, 1)
            return self.teal_keep_fractions()

        for _ in range(iters):
            for li in range(self.L):
                for k in range(4):
                    logt[li][k] = 0.5 * (lo[li][k] + hi[li][k])
            fr = fractions()
            for li in range(self.L):
                for k in range(4):
                    if fr[li][k] > target:
                        lo[li][k] = logt[li][k]
                    else:
                        hi[li][k] = logt[li][k]
        for li in range(self.L):
            for k in range(4):
                logt[li][k] = 0.5 * (lo[li][k] + hi[li][k])
        self.teal_calib_rounds = 0
        gain = [[2.0] * 4 for _ in range(self.L)]
        err = [[0.0] * 4 for _ in range(self.L)]
        for r in range(refine + 1):  # the thresholds kept are the ones last measured
            fr = fractions()
            self.teal_calib_worst = max(abs(f - target) for row in fr for f in row)
            if self.teal_calib_worst <= tol or r == refine:
                break
            self.teal_calib_rounds += 1
            for li in range(self.L):
                for k in range(4):
                    e = fr[li][k] - target
                    if e * err[li][k] < 0:  # overshot: halve this threshold's step
                        gain[li][k] *= 0.5
                    elif e * err[li][k] > 0:  # still short: let it grow back
                        gain[li][k] = min(2.0, 1.5 * gain[li][k])
                    err[li][k] = e
                    logt[li][k] += max(-1.0, min(1.0, gain[li][k] * e))

    # ---------------------------------------------------------------- timing
    def time_blocks(self, run, blocks, block_steps):
        """The pages' protocol: one warm-up block (discarded), then `blocks`
        blocks of `block_steps` steps with an event at each boundary on the
        library's stream.  `run(i0, count)` enqueues steps i0..i0+count-1.
        Returns the per-block µs per step, ascending."""
        torch = self.torch
        run(0, block_steps)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
        ev[0].record(self.stream)
        for b in range(blocks):
            run((1 + b) * block_steps, block_steps)
            ev[b + 1].record(self.stream)
        torch.cuda.synchronize()
        return sorted(ev[b].elapsed_time(ev[b + 1]) * 1e3 / block_steps for b in range(blocks))

    def cell(self, n, k_keep, mode):
        args = self.args
        flags = self.mode_flags(mode)
        ragged = mode.startswith("catekv")
        if flags & self.sd.SD_PROJ_TEAL:
            self.teal_calibrate(n, k_keep, flags)
        self.reset(n, k_keep, ragged)
        blk = self.time_blocks(lambda i0, c: self.run_steps(n + i0, flags, c), args.blocks,
                               args.block_steps)
        us = statistics.median(blk)
        kept = self.wl.d_ff
        if flags & self.sd.SD_MLP_SPARSE:
            kept = sum(int(m.sum()) for m in self.MASK) / self.L
        base = k_keep if flags & self.sd.SD_KV_SPARSE else n
        if ragged:  # mean over layers and KV heads of the per-head kept rows
            base = sum(sum(k) for k in self.ragged_keep) / (self.L * self.wl.n_kv_heads)
        # mean rows read over the timed steps (the warm-up block came first)
        n_read = base + args.block_steps + (args.blocks * args.block_steps - 1) / 2.0 + 1
        out = dict(context=n, mode=mode, us=us, us_min=blk[0], us_max=blk[-1])
        if ragged:
            out["kv_keep_fraction"] = base / n
        if flags & self.sd.SD_PROJ_TEAL:
            b, f = self.teal_step_bytes(n_read, self.teal_keep_fractions())
            out.update(teal_keep=f, teal_calib_worst=self.teal_calib_worst,
                       teal_calib_rounds=self.teal_calib_rounds)
        else:
            b = self.step_bytes(n_read, kept)
            out["n_kept_mean"] = kept
        out.update(bytes=b, gbs=b / us / 1e3, frac=b / us / 1e3 / HBM_PEAK_GBS)
        return out

    def headline(self, n, k_keep, mode):
        """The contract's timed region: W untimed steps, then exactly K steps
        between a device synchronize and events on both sides."""
        torch, args = self.torch, self.args
        flags = self.mode_flags(mode)
        self.reset(n, k_keep)
        self.run_steps(n, flags, args.warmup)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        self.run_steps(n + args.warmup, flags, args.steps)
        e1.record(self.stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        kept = sum(int(m.sum()) for m in self.MASK) / self.L if flags & self.sd.SD_MLP_SPARSE \
            else self.wl.d_ff
        base = k_keep if flags & self.sd.SD_KV_SPARSE else n
        n_read = base + args.warmup + (args.steps - 1) / 2.0 + 1
        b = self.step_bytes(n_read, kept)
        return dict(ms=ms, bytes=b, gbs=b / ms / 1e6, frac=b / ms / 1e6 / HBM_PEAK_GBS,
                    n_kept_mean=kept)

    def profile_cell(self, n, k_keep, mode):
        """Per-kernel event timing of the same steps (library profiler: events
        attached to each dispatch on its stream)."""
        torch, sd, args = self.torch, self.sd, self.args
        flags = self.mode_flags(mode)
        self.reset(n, k_keep)
        self.run_steps(n, flags, args.warmup)
        torch.cuda.synchronize()
        sd.sd_profile_start()
        self.run_steps(n + args.warmup, flags, args.steps)
        stats = sd.sd_profile_stop()
        kept = sum(int(m.sum()) for m in self.MASK) / self.L if flags & sd.SD_MLP_SPARSE \
            else self.wl.d_ff
        wl = self.wl
        d, dh = wl.d_model, wl.head_dim
        base = k_keep if flags & sd.SD_KV_SPARSE else n
        n_read = base + args.warmup + (args.steps - 1) / 2.0 + 1
        alg = {  # algorithmic HBM bytes per launch of each kernel
            "qkv_rope_append": 2 * d * wl.qkv_out,
            "o_residual": 2 * d * wl.n_q_heads * dh,
            "cats_gate_up": 2 * d * wl.d_ff + 2 * d * kept,
            "cats_down": 2 * d * kept,
            "attn_partial": n_read * 2 * wl.n_kv_heads * dh * 2,
        }
        if flags & sd.SD_PROJ_TEAL:  # kept rows of each projection (mean keep per input)
            fr = self.teal_keep_fractions()
            f = [sum(x[k] for x in fr) / len(fr) for k in range(4)]
            qd = wl.n_q_heads * dh
            alg.update(teal_qkv=2 * d * wl.qkv_out * f[0], teal_o=2 * qd * d * f[1],
                       teal_gate_up=4 * d * wl.d_ff * f[2], teal_down=2 * wl.d_ff * d * f[3])
        out = {}
        for name, (launches, tot) in stats.items():
            avg_us = tot / launches * 1e3
            e = dict(launches=launches, avg_us=avg_us, total_ms=tot)
            if name in alg:
                e["alg_bytes"] = alg[name]
                e["gbs"] = alg[name] / (avg_us * 1e-6) / 1e9
                e["frac"] = e["gbs"] / HBM_PEAK_GBS
            out[name] = e
        return out

    def read_ceiling(self, nbytes=4 << 30, reps=10):
        """GB/s of one plain read of a resident nbytes buffer (sd_stream_read,
        the library's own read-only kernel)."""
        torch, sd = self.torch, self.sd
        buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.dev)
        out = torch.empty(sd.SD_STREAM_BLOCKS, dtype=torch.int32, device=self.dev)
        sd.sd_stream_read(buf, nbytes, out)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(reps):
            sd.sd_stream_read(buf, nbytes, out)
        e1.record(self.stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        del buf, out
        torch.cuda.empty_cache()
        return nbytes / ms / 1e6

    def launch_ceiling(self, read_gbs, layers=8, passes=5):
        """Cost of a kernel boundary between streaming launches: sd_stream_read
        over the four weight streams of a composed layer (QKV, O, gate + up at
        50% kept, down at 50% kept), `layers` sets of distinct buffers launched
        back to back on one stream; the time beyond the bytes at the read
        ceiling, per launch."""
        torch, sd, wl = self.torch, self.sd, self.wl
        d, ff = wl.d_model, wl.d_ff
        sizes = [(wl.n_q_heads + 2 * wl.n_kv_heads) * wl.head_dim * d * 2, d * d * 2,
                 int(1.5 * ff * d * 2), int(0.5 * ff * d * 2)]
        sizes = [s // 8192 * 8192 for s in sizes]
        bufs = [torch.zeros(s, dtype=torch.uint8, device=self.dev) for _ in range(layers)
                for s in sizes]
        out = torch.empty(sd.SD_STREAM_BLOCKS, dtype=torch.int32, device=self.dev)
        total = sum(b.numel() for b in bufs)
        times = []
        for it in range(passes + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            for b in bufs:
                sd.sd_stream_read(b, b.numel(), out)
            e1.record(self.stream)
            torch.cuda.synchronize()
            if it:
                times.append(e0.elapsed_time(e1) * 1e3)
        del bufs, out
        torch.cuda.empty_cache()
        us = sorted(times)[len(times) // 2]
        n = layers * len(sizes)
        return dict(launches=n, mb=round(total / 1e6, 1), us=round(us, 1),
                    gbs=round(total / us / 1e3, 1),
                    per_launch_us=round((us - total / read_gbs / 1e3) / n, 2))

    def copy_ceiling(self, nbytes=1 << 30, reps=10):
        """GB/s (read + write) of a plain device-to-device copy of nbytes."""
        torch = self.torch
        src = torch.ones(nbytes, dtype=torch.uint8, device=self.dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        del src, dst
        return 2 * nbytes / ms / 1e6


# ------------------------------------------------------------------- legs
def crossing(stack, sweep):
    """[Cross] §4.3 on this GPU: the measured CATS-vs-KV latency crossing
    (linear interpolation between the bracketing sweep contexts), the latency
    model of the sweep (bw_eff from the dense step's time against its bytes,
    each branch's kernel cost c_X beyond byte time), and from it the byte
    crossover n* and the cost-aware prediction n_lat = n* - (c_P - c_KV)/s,
    all through the library's host calls."""
    sd = stack.sd
    ctx = sorted({c["context"] for c in sweep if c["mode"] in HEAD_MODES})
    by = {(c["context"], c["mode"]): c for c in sweep}
    if len(ctx) < 2 or any((n, m) not in by for n in ctx for m in HEAD_MODES):
        return None
    t = {m: [by[(n, m)]["us"] * 1e-6 for n in ctx] for m in HEAD_MODES}
    b = {m: [by[(n, m)]["bytes"] for n in ctx] for m in HEAD_MODES}
    bw, (c_dense, c_cats, c_kv, c_both) = sd.sd_latency_fit(
        b["dense"], t["dense"], [b["dense"], b["cats"], b["kv"], b["both"]],
        [t["dense"], t["cats"], t["kv"], t["both"]])
    r_p = statistics.mean(by[(n, "cats")]["n_kept_mean"] for n in ctx) / stack.wl.d_ff
    rec = sd.sd_byte_account(stack.dims, stack.L, float(ctx[-1]), r_p, stack.wl.keep_ratio, 2.0,
                             2.0, sd.SD_PROJ_CATS, 0.0, latency=(bw, c_cats, c_kv))
    rec50 = sd.sd_byte_account(stack.dims, stack.L, float(ctx[-1]), 0.5, stack.wl.keep_ratio,
                               2.0, 2.0, sd.SD_PROJ_CATS)
    meas = sd.sd_latency_crossing(ctx, t["cats"], t["kv"])
    dense_kv = sd.sd_latency_crossing(ctx, t["dense"], t["kv"])
    fastest = {n: min(HEAD_MODES, key=lambda m: by[(n, m)]["us"]) for n in ctx}
    return dict(
        measured_cats_vs_kv_tokens=None if math.isnan(meas) else meas,
        n_star_tokens=rec.n_star, n_star_at_half_keep_tokens=rec50.n_star,
        n_lat_tokens=rec.n_lat, gap_per_k_us=rec.gap_per_k * 1e6,
        bw_eff_gbs=bw / 1e9, cats_keep=r_p,
        cost_us=dict(dense=c_dense * 1e6, cats=c_cats * 1e6, kv=c_kv * 1e6, both=c_both * 1e6),
        dense_vs_kv_tokens=None if math.isnan(dense_kv) else dense_kv,
        fastest_mode={str(n): m for n, m in fastest.items()},
        method=("t_X = bytes_X / bw_eff + c_X; bw_eff = inverse least-squares slope of the "
                "dense times against their bytes; c_X = mean excess of mode X over byte time; "
                "measured crossing = linear interpolation of t_CATS - t_KV between the "
                "bracketing contexts"))


def latency_gate(stack, sweep):
    """The lookup table of the latency gate ([Cross] §3.3 "Dispatch and
    batching"), by the library's sd_latency_gate: for each timed context and
    decode length T, the mode with the least total time, T steps plus its
    one-time selection.  Every timed mode is admitted: admissibility is a
    quality test that needs trained weights and real text."""
    out = []
    for n in sorted({c["context"] for c in sweep}):
        cells = [c for c in sweep if c["context"] == n]
        t_step = [c["us"] * 1e-6 for c in cells]
        t_once = [(c.get("select_ms") or 0.0) * 1e-3 for c in cells]
        for T in GATE_HORIZONS:
            best = stack.sd.sd_latency_gate(t_step, t_once, T)
            out.append(dict(context=n, horizon=T, best=cells[best]["mode"],
                            total_ms={c["mode"]: round(1e3 * (T * a + o), 2)
                                      for c, a, o in zip(cells, t_step, t_once)}))
    return out


def single_layer_cells(stack, copies=4):
    """The single-layer cells of the 8B-class layer ([Cross] §4.1, §5.2): 8K
    dense, 32K KV branch at 16% keep with 64 planted keys (with the
    selection's cost and its payback), 4K CATS at sparsity 0.5 and 0.7 beside
    dense.  A step is one layer; `copies` independent layers (weights and
    caches) are stepped in turn, so each layer's bytes (about 0.45 GB) come
    back only after 1.8 GB of others and the 256 MB Infinity Cache cannot
    serve them."""
    import torch
    sd, wl, args = stack.sd, stack.synth.L8B_KV_32K, stack.args
    from synth import device as sdev
    dev, dims = stack.dev, stack.dims
    blocks, bs = args.blocks, args.block_steps
    grow = (1 + blocks) * bs + 8
    out = []

    def mk_layers(n, cap, K, V, KS, VS, cap_sel, thr):
        ls = []
        for i in range(copies):
            W = stack.W[i]
            ls.append((sd.sd_layer * 1)(sd.sd_layer(
                W["attn_norm"].data_ptr(), W["w_qkv"].data_ptr(), W["w_o"].data_ptr(),
                W["mlp_norm"].data_ptr(), W["w_gate"].data_ptr(), W["w_up"].data_ptr(),
                W["w_down_t"].data_ptr(), thr[i], 0, K[i].data_ptr(), V[i].data_ptr(), cap, n,
                None if KS is None else KS[i].data_ptr(),
                None if VS is None else VS[i].data_ptr(), cap_sel, 0, stack.MASK[i].data_ptr())))
            ls[-1][0].w_down_b = W["w_down_b"].data_ptr()
        return ls

    def run_cell(ls, n, k_keep, flags):
        for L in ls:
            L[0].n_full, L[0].n_sel = n, k_keep
        h = stack.h0.clone()

        def run(i0, count):
            for i in range(i0, i0 + count):
                sd.sd_decode_step(dims, ls[i % copies], n + i // copies, h, flags, stack.ws)
        blk = stack.time_blocks(run, blocks, bs)
        return statistics.median(blk), blk[0], blk[-1]

    def record(name, n, mode, us, lo, hi, n_read, kept, **extra):
        b = stack.step_bytes(n_read, kept, layers=1)
        r = dict(cell=name, context=n, mode=mode, us=us, us_min=lo, us_max=hi, bytes=b,
                 gbs=b / us / 1e3, frac=b / us / 1e3 / HBM_PEAK_GBS, **extra)
        out.append(r)
        note("cell", rnd(r))
        return r

    # mean rows each copy reads over the timed steps
    def rows(base):
        return base + bs / copies + (blocks * bs / copies - 1) / 2.0 + 1

    # C2: 8K dense, on the stack's own first layers (their first 8192 rows)
    n = 8192
    ls = mk_layers(n, stack.cap_full, stack.K, stack.V, None, None, 0, [-1.0] * copies)
    us, lo, hi = run_cell(ls, n, 0, 0)
    record("8b-layer-dense-ctx8192", n, "dense", us, lo, hi, rows(n), wl.d_ff)

    # C3: 32K, KV branch at 16% keep, 64 planted keys, own caches per copy
    n = 32768
    k_keep = int(math.floor(0.16 * n))
    cap, cap_sel = n + grow + 64, k_keep + grow + 64
    K, V, KS, VS, planted = [], [], [], [], []
    for i in range(copies):
        k, v = sdev.kv_cache(wl, i, n, cap, dev)
        planted.append(sdev.plant_keys(wl, i, k, n, stack.QW[i], wl.n_planted))
        K.append(k)
        V.append(v)
        KS.append(torch.zeros(wl.n_kv_heads, cap_sel, wl.head_dim, dtype=torch.bfloat16,
                              device=dev))
        VS.append(torch.zeros_like(KS[-1]))
    scores = torch.empty(wl.n_kv_heads, n, device=dev)
    idx = torch.empty(wl.n_kv_heads, k_keep, dtype=torch.int32, device=dev)
    sel_ms, recall = [], []
    for i in range(copies):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stack.stream)
        sd.sd_select_kv(dims, K[i], V[i], cap, n, stack.QW[i], wl.window, wl.n_sink, k_keep,
                        scores, idx, KS[i], VS[i], cap_sel, 0, stack.ws)
        e1.record(stack.stream)
        torch.cuda.synchronize()
        sel_ms.append(e0.elapsed_time(e1))
        got = idx.cpu()
        p = planted[i]
        recall.append(min(int(torch.isin(p, got[h].long()).sum()) for h in range(wl.n_kv_heads)))
    ls = mk_layers(n, cap, K, V, KS, VS, cap_sel, [-1.0] * copies)
    us_d, lo, hi = run_cell(ls, n, k_keep, 0)
    dense = record("8b-layer-dense-ctx32768", n, "dense", us_d, lo, hi, rows(n), wl.d_ff)
    us_k, lo, hi = run_cell(ls, n, k_keep, sd.SD_KV_SPARSE)
    t_sel = statistics.median(sel_ms) * 1e3
    record("8b-layer-kv16-ctx32768", n, "kv", us_k, lo, hi, rows(k_keep), wl.d_ff,
           select_us=t_sel, planted_recall_min=f"{min(recall)}/{wl.n_planted}",
           payback_steps=t_sel / (dense["us"] - us_k) if dense["us"] > us_k else None)
    del K, V, KS, VS, scores, idx, ls
    torch.cuda.empty_cache()

    # C4: 4K, CATS at sparsity 0.5 and 0.7 (per-copy calibrated thresholds) beside dense
    n = 4096
    ls = mk_layers(n, stack.cap_full, stack.K, stack.V, None, None, 0, [-1.0] * copies)
    us, lo, hi = run_cell(ls, n, 0, 0)
    record("8b-layer-dense-ctx4096", n, "dense", us, lo, hi, rows(n), wl.d_ff)
    for s in (0.5, 0.7):
        thr = stack.calibrate(range(copies), s)
        for i, L in enumerate(ls):
            L[0].cats_threshold = thr[i]
        us, lo, hi = run_cell(ls, n, 0, sd.SD_MLP_SPARSE)
        kept = sum(int(stack.MASK[i].sum()) for i in range(copies)) / copies
        record(f"8b-layer-cats{int(s * 10)}-ctx4096", n, f"cats s={s}", us, lo, hi, rows(n),
               kept, n_kept_mean=kept, realized_sparsity=1 - kept / wl.d_ff)
    return dict(copies=copies,
                cache_defeat=(f"{copies} independent layers stepped in turn (about "
                              f"{copies * 0.45:.1f} GB between reuses of one layer's bytes)"),
                cells=out)


def attention_baselines(stack, n, window_ratio=0.3, steps=4, warmup=1):
    """[Cross] §4.4 on this GPU: the same sink-plus-recent window (30% of
    the context, 4 sinks, read in place) against dense decoding whose
    attention runs split-K, fused (one workgroup per query head, no
    split-K) or masked (scores over every allocated row, softmax, P.V;
    K and V read once per query head)."""
    torch, sd, wl = stack.torch, stack.sd, stack.wl
    win = int(math.floor(window_ratio * n))
    for L in stack.layers:
        L.window_keep = win
        L.window_sink = wl.n_sink
    paths = {"split-K": 0, "fused": sd.SD_ATTN_FUSED, "masked": sd.SD_ATTN_MASKED,
             "window (split-K)": sd.SD_KV_WINDOW}
    attn_kinds = ("attn_partial", "attn_combine", "masked_scores", "masked_softmax",
                  "masked_pv")
    out = {}
    for name, flags in paths.items():
        stack.reset(n, 0)
        stack.run_steps(n, flags, warmup)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stack.stream)
        stack.run_steps(n + warmup, flags, steps)
        e1.record(stack.stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        stack.reset(n, 0)
        sd.sd_profile_start()
        stack.run_steps(n, flags, 2)
        stats = sd.sd_profile_stop()
        attn_ms = sum(v[1] for k, v in stats.items() if k in attn_kinds) / (2 * stack.L)
        rows = (win if flags & sd.SD_KV_WINDOW else n) + 1
        kv_bytes = rows * 2 * wl.n_kv_heads * wl.head_dim * 2
        out[name] = dict(us_per_step=ms * 1e3, attn_us_per_layer=attn_ms * 1e3,
                         attn_kv_bytes=kv_bytes, attn_gbs=kv_bytes / attn_ms / 1e6,
                         attn_frac_of_peak=kv_bytes / attn_ms / 1e6 / HBM_PEAK_GBS)
    rec = sd.sd_byte_account(stack.dims, stack.L, float(n), 1.0, win / n, 2.0, 2.0,
                             sd.SD_PROJ_ALL7, 0.0)
    w = out["window (split-K)"]["us_per_step"]
    speedup = {f"vs dense {k}": out[k]["us_per_step"] / w for k in ("split-K", "fused", "masked")}
    return dict(context=n, window_entries=win, sinks=wl.n_sink, paths=out,
                window_speedup=speedup, window_byte_bound=rec.bound_kv)


def batch_caches(stack, n, B, grow):
    """B sequences of context n for the batched step: each sequence's own
    synthetic caches per layer (room for `grow` more rows), its own one-time
    selection at keep ratio wl.keep_ratio into gathered buffers, and its own
    hidden state.  Returns (tensors to keep alive, sd_seq_kv array [B * L],
    sequence-major, k_keep, hidden states [B, d])."""
    torch, sd, wl = stack.torch, stack.sd, stack.wl
    from synth import device as sdev
    cap, k_keep = n + grow + 64, int(math.floor(wl.keep_ratio * n))
    cap_sel = k_keep + grow + 64
    keep, kvs = [], []
    scores = torch.empty(wl.n_kv_heads, n, device=stack.dev)
    idx = torch.empty(wl.n_kv_heads * n, dtype=torch.int32, device=stack.dev)
    sws = torch.empty(sd.sd_workspace_bytes(stack.dims, cap, wl.window), dtype=torch.uint8,
                      device=stack.dev)
    for b in range(B):
        for li in range(stack.L):
            seed = li + 1000 * (b + 1)
            k, v = sdev.kv_cache(wl, seed, n, cap, stack.dev)
            ks = torch.zeros(wl.n_kv_heads, cap_sel, wl.head_dim, dtype=torch.bfloat16,
                             device=stack.dev)
            vs = torch.zeros_like(ks)
            sd.sd_select_kv(stack.dims, k, v, cap, n, sdev.window_queries(wl, seed, stack.dev),
                            wl.window, wl.n_sink, k_keep, scores, idx, ks, vs, cap_sel, 0, sws)
            keep.append((k, v, ks, vs))
            kvs.append(sd.sd_seq_kv(k.data_ptr(), v.data_ptr(), cap, n, ks.data_ptr(),
                                    vs.data_ptr(), cap_sel, k_keep))
    kv = (sd.sd_seq_kv * (B * stack.L))(*kvs)
    h0 = torch.stack([sdev.hidden(wl, b, stack.dev) for b in range(B)])
    torch.cuda.synchronize()
    return keep, kv, k_keep, h0


def batch_cells(stack, n, B, modes, matrix_cores=False):
    """Batched decode ([Cross] §3.3 "Dispatch and batching", §4.4
    "Batching"): B sequences of context n, each with its own synthetic
    caches, selection and hidden state, stepped together so that every
    weight row is read once per step.  Per mode: µs per step (median block
    of a shorter protocol: blocks of a fifth of the sweep's length),
    tokens/s, algorithmic GB/s (weights once, the union's up and down rows
    under CATS, every sequence's cache rows), the measured union fraction
    u_B of the CATS masks, and per-kernel times of one more block (library
    profiler).  matrix_cores: the projections on the matrix cores (tile
    weights), which read up and down whole."""
    torch, sd, wl, args = stack.torch, stack.sd, stack.wl, stack.args
    bs = max(1, args.block_steps // 5)
    grow = (1 + args.blocks) * bs + 8
    keep, kv, k_keep, h0 = batch_caches(stack, n, B, grow)
    hid = h0.clone()
    ws = torch.empty(sd.sd_batch_workspace_bytes(stack.dims, B), dtype=torch.uint8,
                     device=stack.dev)
    d, dh = wl.d_model, wl.head_dim
    w_attn = 2 * (d * wl.qkv_out + wl.n_q_heads * dh * d)
    row = 2 * wl.n_kv_heads * dh * 2
    out = []
    for mode in modes:
        flags = stack.mode_flags(mode) | (sd.SD_MATRIX_CORES if matrix_cores else 0)
        for c in kv:
            c.n_full, c.n_sel = n, k_keep
        hid.copy_(h0)
        pos = [n] * B

        def run(i0, count):
            for _ in range(count):
                sd.sd_decode_step_batch(stack.dims, stack.layers, kv, pos, hid, flags, ws)
                for b in range(B):
                    pos[b] += 1

        blk = stack.time_blocks(run, args.blocks, bs)
        us = statistics.median(blk)
        u = 1.0
        if flags & sd.SD_MLP_SPARSE:
            u = sum(float(m.float().mean()) for m in stack.MASK) / stack.L
        base = k_keep if flags & sd.SD_KV_SPARSE else n
        n_read = base + bs + (args.blocks * bs - 1) / 2.0 + 1
        b_step = stack.L * (w_attn + 2 * d * wl.d_ff * (1 + 2 * u) + B * row * n_read)
        # per-kernel times of one more block; bytes as the account assigns them
        torch.cuda.synchronize()
        sd.sd_profile_start()
        run(0, bs)
        stats = sd.sd_profile_stop()
        qd = wl.n_q_heads * dh
        alg = {"batch_qkv": 2 * d * wl.qkv_out, "batch_o": 2 * qd * d,
               "batch_gate_up": 2 * d * wl.d_ff * (1 + u), "batch_down": 2 * d * wl.d_ff * u,
               "cats_down": 2 * d * wl.d_ff * u,
               "attn_partial": B * row * (n_read + bs)}
        kern = {}
        for name, (launches, tot) in stats.items():
            avg = tot / launches * 1e3
            e = dict(launches=launches, avg_us=avg)
            if name in alg:
                e["gbs"] = alg[name] / (avg * 1e-6) / 1e9
                e["frac"] = e["gbs"] / HBM_PEAK_GBS
            kern[name] = e
        out.append(dict(context=n, batch=B, mode=mode,
                        path="matrix_cores" if matrix_cores else "vector", us=us, us_min=blk[0],
                        us_max=blk[-1], tokens_per_s=B / (us * 1e-6), bytes=b_step,
                        gbs=b_step / us / 1e3, frac=b_step / us / 1e3 / HBM_PEAK_GBS,
                        union_fraction=u if flags & sd.SD_MLP_SPARSE else None, kernels=kern))
    del keep, kv, ws
    torch.cuda.empty_cache()
    return out


# library profiler kind -> rocprofv3 kernel name, source file, and a pattern on
# rocprofv3's full (templated) kernel name where one kernel serves several kinds
KERNEL_SOURCES = {
    "qkv_rope_append": dict(rocprof="qkv_rope_append_kernel", src="gemv.hip"),
    "attn_partial": dict(rocprof="attn_kernel", src="attn.hip"),
    "attn_combine": dict(rocprof="attn_merge_kernel", src="attn.hip"),
    "o_residual": dict(rocprof="o_residual_kernel", src="gemv.hip"),
    "cats_gate_up": dict(rocprof="gate_kernel", src="gemv.hip",
                         match=r"gate_kernel<[^<>]*false, \d+>"),  # not the calibration gate
    # the step's down projection over column blocks (after the CATS gate or a
    # dense one; after TEAL's gate and up), partial sums added in the launch
    "cats_down": dict(rocprof="teal_kernel", src="teal.hip",
                      match=r"teal_kernel<unsigned short, false, 5,"),
    "teal_down": dict(rocprof="teal_kernel", src="teal.hip",
                      match=r"teal_kernel<unsigned short, false, 4,"),
    "teal_qkv": dict(rocprof="teal_kernel", src="teal.hip",
                     match=r"teal_kernel<unsigned short, false, 3,"),
    "teal_o": dict(rocprof="teal_kernel", src="teal.hip",
                   match=r"teal_kernel<unsigned short, false, 1,"),
    "teal_gate_up": dict(rocprof="teal_kernel", src="teal.hip",
                         match=r"teal_kernel<unsigned short, true, 2,"),
    # QKV: the RoPE epilogue (3) with 128-dim heads, else the plain store (0);
    # O: the attention merge in its staging (4) with 128-dim heads, else the
    # residual (1) at 16-step slices
    "batch_qkv": dict(rocprof="bmma_kernel", src="batch_mma.hip",
                      match=r"bmma_kernel<8, false, [03],"),
    "batch_o": dict(rocprof="bmma_kernel", src="batch_mma.hip",
                    match=r"bmma_kernel<8, false, (4, \d+|1, 16)>"),
    "batch_gate_up": dict(rocprof="bmma_kernel", src="batch_mma.hip",
                          match=r"bmma_kernel<8, true, 2,"),
    "batch_down": dict(rocprof="bmma_kernel", src="batch_mma.hip",
                       match=r"bmma_kernel<8, false, 1, 32>"),
}


def source_digest(src: str) -> str:
    """Hash of a kernel's source file and the headers every kernel includes."""
    h = hashlib.sha256()
    for f in (src, "common.hpp", "internal.hpp"):
        h.update(open(os.path.join(ROOT, "kv_cache_activation_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def traffic_for(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only
    while the kernel's source is unchanged since the counters were taken."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        rec = json.load(open(TRAFFIC_JSON))["kernels"][kernel]
        if source_digest(KERNEL_SOURCES[kernel]["src"]) != rec["sha256"]:
            return None
        return rec["bytes_per_launch"]
    except Exception:
        return None


def pmc_summary(fetch_csv: str, write_csv: str, copy_bytes: int, out: str) -> None:
    """Per-kernel HBM bytes per dispatch from two rocprofv3 --pmc runs of this
    script (FETCH_SIZE, then WRITE_SIZE, in KiB), each scaled by what the same
    counter reads for the plain device copy of `copy_bytes` bytes that the runs
    start with (--pmc-copy-bytes).  The decode-step launches of a kernel are
    its most frequent grid size (calibration launches differ) among the
    dispatches whose full kernel name matches the kind's pattern."""
    import collections
    import csv
    import re

    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Correlation_Id"]))
        # the calibration: the first three large copies of the run (later ones,
        # such as the copy-ceiling measurement, move other sizes)
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copy" in r["Kernel_Name"] and float(r["Counter_Value"]) * 1024 > copy_bytes / 4]
        copies = copies[:3]
        if not copies:
            raise SystemExit(f"{path}: no copy-kernel dispatch of about {copy_bytes} bytes found")
        scale = copy_bytes / (sorted(copies)[len(copies) // 2] * 1024)
        per = collections.defaultdict(lambda: collections.defaultdict(list))
        for kind, e in KERNEL_SOURCES.items():
            pat = e.get("match", r"sd::%s\b" % e["rocprof"])
            for r in rows:
                if re.search(r"sd::%s\b" % e["rocprof"], r["Kernel_Name"]) and \
                        re.search(pat, r["Kernel_Name"]):
                    per[kind][r["Grid_Size"]].append(float(r["Counter_Value"]) * 1024 * scale)
        return scale, per

    fs, fetch = load(fetch_csv, "FETCH_SIZE")
    ws, write = load(write_csv, "WRITE_SIZE")
    res = dict(about=("HBM bytes per dispatch of the decode-step kernels, from rocprofv3 --pmc "
                      "FETCH_SIZE and WRITE_SIZE, each scaled by the counter's reading for a "
                      f"plain {copy_bytes}-byte device copy"),
               fetch_scale=fs, write_scale=ws, kernels={})
    for kind, e in KERNEL_SOURCES.items():
        if kind not in fetch or kind not in write:
            continue
        grid = max(fetch[kind], key=lambda g: len(fetch[kind][g]))
        f = fetch[kind][grid]
        w = write[kind].get(grid, [0.0])
        fb, wb = sum(f) / len(f), sum(w) / len(w)
        res["kernels"][kind] = dict(rocprof_name=e["rocprof"], grid_size=int(grid),
                                    dispatches=len(f), fetch_bytes=round(fb),
                                    write_bytes=round(wb), bytes_per_launch=round(fb + wb),
                                    source=e["src"], sha256=source_digest(e["src"]))
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


def trace_summary(csv_path: str, out: str, title: str, cmd: str) -> None:
    """Markdown summary of a rocprofv3 --kernel-trace CSV of this script: per
    library kind (KERNEL_SOURCES), the decode-step launches (the kind's most
    frequent grid size) with their mean, min and max duration, and every
    library kernel's launch count and mean duration."""
    import collections
    import csv
    import re

    rows = [r for r in csv.DictReader(open(csv_path)) if "sd::" in r["Kernel_Name"]]
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # noqa: E731
    lines = [f"# rocprofv3 kernel summary: {title}", "",
             "Command (from the repository root, on one MI355X), then this summary:", "", "```",
             cmd, f"python3 bench.py --trace-summary {csv_path} --trace-out {out} "
             f"--trace-title \"{title}\" --trace-cmd \"<the command above>\"", "```", "",
             "## Decode-step launches per kernel kind", "",
             "Launches of the kind's most frequent grid size (one per layer and step; the "
             "one-time selection and calibration launches have other grids).", "",
             "| kind | kernel | grid (threads) | launches | mean µs | min µs | max µs |",
             "|---|---|---|---|---|---|---|"]
    for kind, e in KERNEL_SOURCES.items():
        pat = e.get("match", r"sd::%s\b" % e["rocprof"])
        sel = [r for r in rows if re.search(r"sd::%s\b" % e["rocprof"], r["Kernel_Name"])
               and re.search(pat, r["Kernel_Name"])]
        if not sel:
            continue
        by = collections.Counter(int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) *
                                 int(r["Grid_Size_Z"]) for r in sel)
        grid = by.most_common(1)[0][0]
        ds = [dur(r) for r in sel
              if int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) == grid]
        lines.append(f"| {kind} | `{e['rocprof']}` | {grid} | {len(ds)} | "
                     f"{sum(ds) / len(ds):.2f} | {min(ds):.2f} | {max(ds):.2f} |")
    lines += ["", "## Every library kernel", "", "| kernel | launches | mean µs | total ms |",
              "|---|---|---|---|"]
    agg = collections.defaultdict(list)
    for r in rows:
        m = re.search(r"sd::(\w+(<[^()]*>)?)", r["Kernel_Name"])
        agg[m.group(1) if m else r["Kernel_Name"]].append(dur(r))
    for name, ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {len(ds)} | {sum(ds) / len(ds):.2f} | {sum(ds) / 1e3:.2f} |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as f:
            f.write(text)
    print(text)


def cpu_baseline(stack, n, seconds):
    """The float64 oracle, timed as it stands on the host cores, on a bounded
    sample of the headline workload: the first layer of the stack (its own
    weights and 128K cache copied to the host), composed mode, repeated until
    `seconds` have passed; per-step time scaled to all layers."""
    import numpy as np

    from oracle import cats as ocats, step as ostep

    wl = stack.wl
    W = {k: v.float().cpu().numpy() for k, v in stack.W[0].items() if k != "w_down_b"}
    reps_cap = 512
    shape = (wl.n_kv_heads, n + reps_cap, wl.head_dim)
    k = np.zeros(shape, np.float32)
    v = np.zeros(shape, np.float32)
    k[:, :n] = stack.K[0][:, :n].float().cpu().numpy()
    v[:, :n] = stack.V[0][:, :n].float().cpu().numpy()
    k_keep = int(math.floor(wl.keep_ratio * n))
    # the rows kept do not change the work; take the first k_keep rows
    ks = np.zeros((wl.n_kv_heads, k_keep + reps_cap, wl.head_dim), np.float32)
    vs = np.zeros_like(ks)
    ks[:, :k_keep] = k[:, :k_keep]
    vs[:, :k_keep] = v[:, :k_keep]
    h = stack.h0.cpu().numpy().astype(np.float64)
    x2 = ostep.rmsnorm(h, W["mlp_norm"], 1e-5)
    t = float(np.median(np.abs(ocats.gate_act(x2, W["w_gate"]).astype(np.float32))))
    layer = ostep.Layer(W["attn_norm"], W["w_qkv"], W["w_o"], W["mlp_norm"], W["w_gate"],
                        W["w_up"], W["w_down_t"], t, k, v, n, ks, vs, k_keep)
    dims = dict(n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                kv_dtype="bf16", eps=1e-5, theta=500000.0)
    reps = 0
    t0 = time.perf_counter()
    while reps < reps_cap - 2 and (reps == 0 or time.perf_counter() - t0 < seconds):
        tr = []
        h = ostep.decode_layer(layer, h, n + reps, kv_sparse=True, mlp_sparse=True, trace=tr,
                               **dims)
        reps += 1
    per_layer = (time.perf_counter() - t0) / reps
    kept = float(tr[0]["mask"].sum())
    per_step = per_layer * stack.L
    b = stack.step_bytes(k_keep + reps / 2.0 + 1, kept)
    cores, blas, single = 1, None, None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        info = threadpool_info()
        cores = max((p.get("num_threads", 1) for p in info), default=1)
        blas = ",".join(sorted({str(p.get("internal_api")) for p in info})) or None
        r1, t1 = 0, time.perf_counter()
        with threadpool_limits(limits=1):
            while reps + r1 < reps_cap - 2 and (r1 == 0 or time.perf_counter() - t1 < seconds / 2):
                h = ostep.decode_layer(layer, h, n + reps + r1, kv_sparse=True, mlp_sparse=True,
                                       **dims)
                r1 += 1
        single = b / ((time.perf_counter() - t1) / r1 * stack.L) / 1e9
    except ImportError:
        pass
    return dict(value=b / per_step / 1e9, unit="GB/s", cores=int(cores), kind="oracle",
                ms_per_step=per_step * 1e3, blas=blas,
                affinity_cores=len(os.sched_getaffinity(0)), single_thread_gbs=single,
                sample=(f"float64 numpy oracle, layer 0 of the stack at context {n}, composed "
                        f"mode, {reps} decode steps of that layer in {per_layer * reps:.1f} s, "
                        f"scaled x{stack.L} layers"))


def headline_line(args, stack, head, roof, cpu, sweep, cross, wall_s):
    """The one compact JSON record printed last on stdout."""
    n_head = max(stack.contexts)
    ctx = sorted({c["context"] for c in sweep})
    by = {(c["context"], c["mode"]): c for c in sweep}
    table = {m: [round(by[(n, m)]["us"], 1) if (n, m) in by else None for n in ctx]
             for m in HEAD_MODES}
    frac = {m: [round(by[(n, m)]["frac"], 3) if (n, m) in by else None for n in ctx]
            for m in HEAD_MODES}
    return dict(
        metric=METRIC, value=round(head["gbs"], 1), unit="GB/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(head["ms"], 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=stack.wl.name if n_head == 131072 and stack.L == 32
                    else f"8b-{stack.L}layer-bf16-both-ctx{n_head}",
                    layers=stack.L, context=n_head, mode="both", kv_keep=stack.wl.keep_ratio,
                    cats_sparsity=0.5, storage="bf16", accumulate="f32",
                    hbm_frac=round(head["frac"], 4), bytes_per_step=round(head["bytes"])),
        roofline=roof,
        cpu_baseline=None if cpu is None else dict(
            value=round(cpu["value"], 3), unit="GB/s", cores=cpu["cores"], kind="oracle",
            sample=cpu["sample"]),
        sweep=dict(ctx=ctx, us=table, frac=frac,
                   protocol=f"median of {args.blocks} blocks x {args.block_steps} steps after "
                            f"a {args.block_steps}-step warm-up block"),
        crossing=None if cross is None else dict(
            measured_k=None if cross["measured_cats_vs_kv_tokens"] is None
            else round(cross["measured_cats_vs_kv_tokens"] / 1024, 2),
            n_star_k=round(cross["n_star_tokens"] / 1024, 2),
            n_lat_k=round(cross["n_lat_tokens"] / 1024, 2),
            bw_eff_gbs=round(cross["bw_eff_gbs"], 1),
            cost_us={k: round(v, 1) for k, v in cross["cost_us"].items()}),
        wall_s=wall_s,
    )


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.pmc_copy_bytes, args.pmc_out)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.trace_out, args.trace_title, args.trace_cmd)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported by this build "
              "(the sharded multi-GPU path is a design note only)", file=sys.stderr)
        sys.exit(2)
    legs = set(x for x in args.legs.split(",") if x)
    unknown = legs - set(LEGS)
    if unknown:
        raise SystemExit(f"unknown legs {sorted(unknown)}; known: {LEGS}")
    import torch
    if args.pmc_copy_bytes:
        src = torch.ones(args.pmc_copy_bytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    t_start = time.perf_counter()
    stack = Stack(args)
    note("setup", dict(layers=stack.L, contexts=stack.contexts,
                       s=round(time.perf_counter() - t_start, 1)))
    full = dict(protocol=dict(blocks=args.blocks, block_steps=args.block_steps,
                              warmup_block_steps=args.block_steps,
                              headline_warmup=args.warmup, headline_steps=args.steps))
    sweep = []
    sel_ms = {}
    n_head = max(stack.contexts)
    k_head = int(math.floor(stack.wl.keep_ratio * n_head))
    for n in stack.contexts:
        if "sweep" not in legs and (n != n_head or "head" not in legs):
            continue
        secs, k_keep = stack.select(n)
        sel_ms[n] = secs * 1e3
        modes = [m for m in HEAD_MODES if m in args.modes.split(",")]
        for mode in (modes if "sweep" in legs else ("both",)):
            c = stack.cell(n, k_keep, mode)
            c["select_ms"] = sel_ms[n] if stack.mode_flags(mode) & stack.sd.SD_KV_SPARSE else None
            sweep.append(c)
            print(f"# n={n:6d} {mode:5s} {c['us']:9.1f} us/step (blocks {c['us_min']:.1f}.."
                  f"{c['us_max']:.1f}) {c['gbs']:7.1f} GB/s ({100 * c['frac']:.1f}% of peak)",
                  flush=True)
    head = roof = None
    if "head" in legs:
        # the headline cell: the contract's W + K steps (the selection of n_head in place)
        head = stack.headline(n_head, k_head, "both")
        print(f"# headline n={n_head} both: {head['ms'] * 1e3:.1f} us/step over {args.steps} "
              f"steps, {head['gbs']:.1f} GB/s ({100 * head['frac']:.1f}% of peak)", flush=True)
        kern = stack.profile_cell(n_head, k_head, "both")
        dom = max((k for k in kern if "alg_bytes" in kern[k]), key=lambda k: kern[k]["total_ms"])
        dk = kern[dom]
        roof = dict(bound="hbm", achieved=round(dk["gbs"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(dk["frac"], 4), traffic=traffic_for(dom),
                    kernel=KERNEL_SOURCES[dom]["rocprof"], avg_us=round(dk["avg_us"], 2),
                    alg_bytes_per_launch=dk["alg_bytes"])
        full["kernels"] = rnd(kern)
        note("kernels", {k: rnd({kk: e[kk] for kk in ("launches", "avg_us", "gbs", "frac")
                                 if kk in e}, 3) for k, e in kern.items()})
    cross = crossing(stack, sweep) if "sweep" in legs else None
    if cross:
        full["crossing"] = rnd(cross)
        note("crossing", rnd({k: v for k, v in cross.items() if k != "method"}, 1))
    if "sweep" in legs and all((n_head, m) in {(c["context"], c["mode"]) for c in sweep}
                               for m in ("dense", "kv")):
        gate = latency_gate(stack, sweep)
        full["latency_gate"] = gate
        note("latency_gate", {f"{g['context']}/{g['horizon']}": g["best"] for g in gate})
        pay = None
        at = {c["mode"]: c for c in sweep if c["context"] == n_head}
        if at["dense"]["us"] > at["kv"]["us"]:
            pay = sel_ms[n_head] * 1e3 / (at["dense"]["us"] - at["kv"]["us"])
        full["selection"] = dict(select_ms_all_layers=rnd(sel_ms, 2),
                                 payback_steps_at_head=None if pay is None else round(pay, 1))
        note("selection", full["selection"])
    if "cells" in legs:
        full["single_layer"] = rnd(single_layer_cells(stack))
    extra = []
    if "teal" in legs:
        stack.enable_teal()
        for n in sorted(int(c) for c in args.teal_contexts.split(",") if c):
            _, k_keep = stack.select(n)
            for mode in [m for m in args.teal_modes.split(",") if m]:
                c = stack.cell(n, k_keep, mode)
                extra.append(c)
                note("teal", rnd(c))
            if n == max(int(c) for c in args.teal_contexts.split(",") if c):
                kt = stack.profile_cell(n, k_keep, "teal+kv")
                full["teal_kernels"] = rnd(kt)
                note("teal_kernels", {k: rnd({kk: e[kk] for kk in ("launches", "avg_us", "gbs",
                                                                   "frac") if kk in e}, 3)
                                      for k, e in kt.items()})
        stack.disable_teal()
    if "catekv" in legs:
        stack.enable_ragged()
        for n in sorted(int(c) for c in args.catekv_contexts.split(",") if c):
            sel_r = stack.select_ragged(n) * 1e3
            for mode in ("catekv", "catekv+cats"):
                c = stack.cell(n, 0, mode)
                c["select_ms"] = sel_r
                extra.append(c)
                note("catekv", rnd(c))
        stack.disable_ragged()
    full["teal_catekv"] = rnd(extra)
    if "baselines" in legs:
        base = attention_baselines(stack, n_head)
        full["attention_baselines"] = rnd(base)
        note("attention_baselines", rnd(dict(
            speedup=base["window_speedup"], bound=base["window_byte_bound"],
            attn_frac={k: v["attn_frac_of_peak"] for k, v in base["paths"].items()}), 3))
    if "batch" in legs and args.batches:
        cells = []
        paths = [p for p in args.batch_paths.split(",") if p]
        if "matrix_cores" in paths:
            stack.enable_tiles()
        for n in [int(c) for c in args.batch_contexts.split(",") if c]:
            for B in [int(b) for b in args.batches.split(",") if b]:
                for path in paths:
                    bmodes = [m for m in args.batch_modes.split(",") if m]
                    for c in batch_cells(stack, n, B, bmodes, path == "matrix_cores"):
                        cells.append(c)
                        note("batch", rnd({k: v for k, v in c.items() if k != "kernels"}, 3))
                        note("batch_kernels", rnd(c["kernels"], 3))
        if "matrix_cores" in paths:
            stack.disable_tiles()
        union = {}
        for B in sorted({c["batch"] for c in cells}):
            us = [c["union_fraction"] for c in cells if c["batch"] == B and c["union_fraction"]]
            u = sum(us) / len(us)
            n_star = stack.sd.sd_byte_crossover_batch(stack.dims, B, u, stack.wl.keep_ratio, 2.0,
                                                      2.0, stack.sd.SD_PROJ_CATS)
            union[str(B)] = dict(measured=round(u, 4), independent=round(1 - 0.5 ** B, 4),
                                 n_star_tokens=round(n_star, 1))
        full["batch"] = dict(cells=rnd(cells), union=union)
        note("batch_union", union)
    cpu = None
    if "cpu" in legs:
        cpu = cpu_baseline(stack, n_head, args.cpu_seconds)
        full["cpu_baseline"] = rnd(cpu)
        note("cpu_baseline", rnd({k: v for k, v in cpu.items() if k != "sample"}, 3))
    full["copy_ceiling_gbs"] = round(stack.copy_ceiling(), 1)
    full["read_ceiling_gbs"] = round(stack.read_ceiling(), 1)
    full["launch_ceiling"] = stack.launch_ceiling(full["read_ceiling_gbs"])
    note("ceilings", dict(read_gbs=full["read_ceiling_gbs"], copy_gbs=full["copy_ceiling_gbs"],
                          launch=full["launch_ceiling"]))
    full["sweep"] = rnd(sweep)
    full["wall_s"] = round(time.perf_counter() - t_start, 1)
    line = None
    if head is not None:
        line = headline_line(args, stack, head, roof, cpu, sweep, cross, full["wall_s"])
        line["read_ceiling_gbs"] = full["read_ceiling_gbs"]
        line["launch_overhead_us"] = full["launch_ceiling"]["per_launch_us"]
        full["headline"] = line
    if args.out:
        with open(args.out, "w") as f:
            json.dump(full, f, indent=1)
    if line is not None:
        print(json.dumps(line, separators=(",", ":")), flush=True)
    else:  # a run without the head leg (profiling runs): no contract line
        note("done", dict(legs=sorted(legs), wall_s=full["wall_s"]))


if __name__ == "__main__":
    main()
