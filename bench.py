#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X.

Workload: 32 stacked 8B-class layers (d 4096, 32/8 heads, head_dim 128, FFN
14336, bf16 weights and caches) with independent N(0, 0.02^2) weights and
synthetic caches (K, V ~ N(0,1) times LogNormal(0, 0.5) channel scales), at
context 2K/8K/32K/64K/128K, in four modes: dense, KV (10% keep, one-time
attention-scored selection), CATS (thresholds for 50% gate sparsity from 256
Gaussian calibration states per layer), and both.  The headline is the
composed step ("both") at 128K.

A step is one call of sd_decode_step through all 32 layers (each layer
appends its key/value row, so the context grows by one per step).  Inputs are
resident in HBM before timing; W warm-up steps, then K timed steps bracketed
by a device synchronize and HIP events on the library's stream.

value = algorithmic HBM bytes per step / time per step (GB/s, 1e9 bytes):
weights read (QKV, O, gate, kept up rows, kept down rows), cached K/V rows
read, and the appended rows written.
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
MODES = ("dense", "kv", "cats", "both", "teal", "teal+kv", "catekv", "catekv+cats")
# CateKV's benchmark setting: 40% of the KV heads adaptive (eta = 1 keeps all
# their entries), the others keep a budget of 2048
CATEKV_RATIO, CATEKV_ETA, CATEKV_BUDGET = 0.4, 1.0, 2048
# decode lengths over which the latency gate charges one-time selection
GATE_HORIZONS = (256, 1024, 4096, 16384)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--contexts", type=str, default="2048,8192,32768,65536,131072")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--modes", type=str, default=",".join(MODES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attn-baselines", action="store_true",
                    help="skip the window-vs-dense-attention-path comparison at the largest context")
    ap.add_argument("--batches", type=str, default="4,8",
                    help="batch sizes of the batched-decode leg (empty: skip it)")
    ap.add_argument("--batch-contexts", type=str, default="8192,32768")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--out", type=str, default="")
    ap.add_argument("--pmc-copy-bytes", type=int, default=0,
                    help="start with three plain device copies of this many bytes (counter "
                         "calibration for rocprofv3 --pmc runs)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter CSVs of this script into "
                         "per-kernel HBM bytes (needs --pmc-copy-bytes of those runs)")
    ap.add_argument("--pmc-out", type=str, default=TRAFFIC_JSON)
    return ap.parse_args()


class Bench:
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
        self.contexts = [int(c) for c in args.contexts.split(",")]
        n_max = max(self.contexts)
        grow = args.warmup + args.steps + 2
        self.cap_full = n_max + grow + 64
        self.cap_sel = int(math.floor(wl.keep_ratio * n_max)) + grow + 64
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
        self.thresholds = self.calibrate()
        layers = []
        for li in range(self.L):
            W = self.W[li]
            layers.append(sd.sd_layer(
                W["attn_norm"].data_ptr(), W["w_qkv"].data_ptr(), W["w_o"].data_ptr(),
                W["mlp_norm"].data_ptr(), W["w_gate"].data_ptr(), W["w_up"].data_ptr(),
                W["w_down_t"].data_ptr(), self.thresholds[li], 0, self.K[li].data_ptr(),
                self.V[li].data_ptr(), self.cap_full, 0, self.KS[li].data_ptr(),
                self.VS[li].data_ptr(), self.cap_sel, 0, self.MASK[li].data_ptr()))
        self.layers = (sd.sd_layer * self.L)(*layers)
        self.ragged = any(m.startswith("catekv") for m in getattr(args, "modes", "").split(","))
        if self.ragged:  # CateKV: one gathered buffer per layer with a budget per KV head
            import ctypes
            self.adaptive = synth.catekv_adaptive(wl, self.L, CATEKV_RATIO)
            self.cap_r = n_max + grow + 64
            self.KR, self.VR, self.RH = [], [], []
            for li in range(self.L):
                self.KR.append(torch.zeros(wl.n_kv_heads, self.cap_r, wl.head_dim,
                                           dtype=torch.bfloat16, device=self.dev))
                self.VR.append(torch.zeros_like(self.KR[-1]))
                self.RH.append((ctypes.c_int32 * wl.n_kv_heads)())
            self.ragged_keep = None
        self.teal = any(m.startswith("teal") for m in getattr(args, "modes", "").split(","))
        if self.teal:  # TEAL mode reads the projections transposed (input-major)
            self.WT, self.TMASK = [], []
            d, qd, ff = wl.d_model, wl.n_q_heads * wl.head_dim, wl.d_ff
            self.teal_sizes = (d, qd, d, ff)
            for li in range(self.L):
                W = self.W[li]
                wt = {k: W[k].t().contiguous() for k in ("w_qkv", "w_o", "w_gate", "w_up")}
                self.WT.append(wt)
                self.TMASK.append(torch.zeros(sum(self.teal_sizes), dtype=torch.uint8,
                                              device=self.dev))
                L = self.layers[li]
                L.w_qkv_t, L.w_o_t = wt["w_qkv"].data_ptr(), wt["w_o"].data_ptr()
                L.w_gate_t, L.w_up_t = wt["w_gate"].data_ptr(), wt["w_up"].data_ptr()
                L.teal_masks_out = self.TMASK[li].data_ptr()
        torch.cuda.synchronize()

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
                li, k = max(((i, j) for i in range(self.L) for j in range(4)),
                            key=lambda ij: abs(fr[ij[0]][ij[1]] - target))
                print(f"# teal calibration n={n}: {r} Newton rounds, worst layer {li} input {k} "
                      f"keeps {fr[li][k]:.4f} at t={math.exp(logt[li][k]):.4g}", flush=True)
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

    def calibrate(self, n_states=256, sparsity=0.5):
        torch, sd = self.torch, self.sd
        from synth import device as sdev
        ws = torch.empty(sd.sd_calibrate_workspace_bytes(self.dims, n_states), dtype=torch.uint8,
                         device=self.dev)
        thr = torch.empty(self.L, device=self.dev)
        for li in range(self.L):
            states = sdev.calibration_states(self.wl, li, n_states, self.dev)
            sd.sd_cats_calibrate(self.dims, states, n_states, self.W[li]["mlp_norm"],
                                 self.W[li]["w_gate"], sparsity, thr[li:li + 1], ws)
        return thr.cpu().tolist()

    def copy_ceiling(self, nbytes=1 << 30, reps=10):
        """GB/s (read + write) of a plain device-to-device copy of nbytes: the
        streaming rate this GPU reaches outside the decode step."""
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

    def step_bytes(self, n_read, n_kept_mean):
        wl = self.wl
        d, dh = wl.d_model, wl.head_dim
        w = 2 * (d * wl.qkv_out + wl.n_q_heads * dh * d + d * wl.d_ff + 2 * d * n_kept_mean)
        row = 2 * wl.n_kv_heads * dh * 2
        return self.L * (w + row * n_read + 2 * row)

    def mode_flags(self, mode):
        sd = self.sd
        return {"dense": 0, "kv": sd.SD_KV_SPARSE, "cats": sd.SD_MLP_SPARSE,
                "both": sd.SD_KV_SPARSE | sd.SD_MLP_SPARSE, "teal": sd.SD_PROJ_TEAL,
                "teal+kv": sd.SD_PROJ_TEAL | sd.SD_KV_SPARSE, "catekv": sd.SD_KV_SPARSE,
                "catekv+cats": sd.SD_KV_SPARSE | sd.SD_MLP_SPARSE}[mode]

    def teal_step_bytes(self, n_read, fr):
        """Algorithmic bytes of a TEAL step: each projection's kept rows (mean
        kept fraction of its input over the layers) plus the cache rows."""
        wl = self.wl
        d, qd, ff = wl.d_model, wl.n_q_heads * wl.head_dim, wl.d_ff
        f = [sum(x[k] for x in fr) / len(fr) for k in range(4)]
        w = 2 * (d * wl.qkv_out * f[0] + qd * d * f[1] + 2 * d * ff * f[2] + ff * d * f[3])
        row = 2 * wl.n_kv_heads * wl.head_dim * 2
        return self.L * (w + row * n_read + 2 * row), f

    def cell(self, n, k_keep, mode):
        torch, args = self.torch, self.args
        flags = self.mode_flags(mode)
        ragged = mode.startswith("catekv")
        if flags & self.sd.SD_PROJ_TEAL:
            self.teal_calibrate(n, k_keep, flags)
        self.reset(n, k_keep, ragged)
        self.run_steps(n, flags, args.warmup)
        torch.cuda.synchronize()
        # the timed steps in up to 4 blocks, an event at each block boundary
        # (on the library's stream, inside the one timed region)
        nblk = max(1, min(4, args.steps))
        cuts = [round(i * args.steps / nblk) for i in range(nblk + 1)]
        ev = [torch.cuda.Event(enable_timing=True) for _ in cuts]
        ev[0].record(self.stream)
        for i in range(nblk):
            self.run_steps(n + args.warmup + cuts[i], flags, cuts[i + 1] - cuts[i])
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[-1]) / args.steps
        blk = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 / (cuts[i + 1] - cuts[i])
                     for i in range(nblk))
        kept = self.wl.d_ff
        if flags & self.sd.SD_MLP_SPARSE:
            kept = sum(int(m.sum()) for m in self.MASK) / self.L
        base = k_keep if flags & self.sd.SD_KV_SPARSE else n
        if ragged:  # mean over layers and KV heads of the per-head kept rows
            base = sum(sum(k) for k in self.ragged_keep) / (self.L * self.wl.n_kv_heads)
        n_read = base + args.warmup + (args.steps - 1) / 2.0 + 1
        extra = {}
        if ragged:
            extra["kv_keep_fraction"] = round(base / n, 4)
        if flags & self.sd.SD_PROJ_TEAL:
            b, f = self.teal_step_bytes(n_read, self.teal_keep_fractions())
            extra = dict(teal_keep=[round(x, 4) for x in f],
                         teal_calib_worst=round(self.teal_calib_worst, 4),
                         teal_calib_rounds=self.teal_calib_rounds)
        else:
            b = self.step_bytes(n_read, kept)
            extra["n_kept_mean"] = kept
        extra["us_per_step_blocks"] = dict(blocks=nblk, min=round(blk[0], 1),
                                           median=round(statistics.median(blk), 1),
                                           max=round(blk[-1], 1))
        return dict(context=n, mode=mode, ms_per_step=ms, us_per_step=ms * 1e3,
                    bytes_per_step=b, gbs=b / ms / 1e6, hbm_frac=b / ms / 1e6 / HBM_PEAK_GBS,
                    kv_rows_read=n_read, **extra)

    def attention_baselines(self, n, window_ratio=0.3, steps=4, warmup=1):
        """[Cross] §4.4 on this GPU: the same sink-plus-recent window (30% of
        the context, 4 sinks, read in place) against dense decoding whose
        attention runs split-K, fused (one workgroup per query head, no
        split-K) or masked (scores over every allocated row, softmax, P.V;
        K and V read once per query head).  Returns per path the step time,
        the attention kernels' time per layer and the bandwidth they reach on
        the K/V bytes attention must read, plus the window's speedups and its
        byte bound from the library's byte account."""
        torch, sd, wl = self.torch, self.sd, self.wl
        win = int(math.floor(window_ratio * n))
        for L in self.layers:
            L.window_keep = win
            L.window_sink = wl.n_sink
        paths = {"split-K": 0, "fused": sd.SD_ATTN_FUSED, "masked": sd.SD_ATTN_MASKED,
                 "window (split-K)": sd.SD_KV_WINDOW}
        attn_kinds = ("attn_partial", "attn_combine", "masked_scores", "masked_softmax",
                      "masked_pv")
        out = {}
        for name, flags in paths.items():
            self.reset(n, 0)
            self.run_steps(n, flags, warmup)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            self.run_steps(n + warmup, flags, steps)
            e1.record(self.stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            self.reset(n, 0)
            sd.sd_profile_start()
            self.run_steps(n, flags, 2)
            stats = sd.sd_profile_stop()
            attn_ms = sum(v[1] for k, v in stats.items() if k in attn_kinds) / (2 * self.L)
            rows = (win if flags & sd.SD_KV_WINDOW else n) + 1
            kv_bytes = rows * 2 * wl.n_kv_heads * wl.head_dim * 2  # K and V rows attention reads
            out[name] = dict(us_per_step=round(ms * 1e3, 1), attn_us_per_layer=round(attn_ms * 1e3, 2),
                             attn_kv_bytes=kv_bytes,
                             attn_gbs=round(kv_bytes / attn_ms / 1e6, 1),
                             attn_frac_of_peak=round(kv_bytes / attn_ms / 1e6 / HBM_PEAK_GBS, 4))
        rec = sd.sd_byte_account(self.dims, self.L, float(n), 1.0, win / n, 2.0, 2.0,
                                 sd.SD_PROJ_ALL7, 0.0)
        w = out["window (split-K)"]["us_per_step"]
        speedup = {f"vs dense {k}": round(out[k]["us_per_step"] / w, 3)
                   for k in ("split-K", "fused", "masked")}
        return dict(context=n, window_entries=win, sinks=wl.n_sink, paths=out,
                    window_speedup=speedup, window_byte_bound=round(rec.bound_kv, 3))

    def batch_cells(self, n, B, modes):
        """Batched decode ([Cross] §3.2 "Dispatch and batching", §4.4
        "Batching"): B sequences of context n, each with its own synthetic
        caches, selection and hidden state, stepped together so that every
        weight row is read once per step.  Per mode: µs per step, tokens/s
        (B per step), algorithmic GB/s (weights once, the union's up and down
        rows under CATS, every sequence's cache rows), and the measured union
        fraction u_B of the CATS masks."""
        torch, sd, wl, args = self.torch, self.sd, self.wl, self.args
        from synth import device as sdev
        grow = args.warmup + args.steps + 2
        cap, k_keep = n + grow + 64, int(math.floor(wl.keep_ratio * n))
        cap_sel = k_keep + grow + 64
        keep, kvs = [], []
        # selection buffers sized for this context
        scores = torch.empty(wl.n_kv_heads, n, device=self.dev)
        idx = torch.empty(wl.n_kv_heads * n, dtype=torch.int32, device=self.dev)
        sws = torch.empty(sd.sd_workspace_bytes(self.dims, cap, wl.window), dtype=torch.uint8,
                          device=self.dev)
        for b in range(B):
            for li in range(self.L):
                seed = li + 1000 * (b + 1)
                k, v = sdev.kv_cache(wl, seed, n, cap, self.dev)
                ks = torch.zeros(wl.n_kv_heads, cap_sel, wl.head_dim, dtype=torch.bfloat16,
                                 device=self.dev)
                vs = torch.zeros_like(ks)
                sd.sd_select_kv(self.dims, k, v, cap, n, sdev.window_queries(wl, seed, self.dev),
                                wl.window, wl.n_sink, k_keep, scores, idx, ks, vs, cap_sel, 0,
                                sws)
                keep.append((k, v, ks, vs))
                kvs.append(sd.sd_seq_kv(k.data_ptr(), v.data_ptr(), cap, n, ks.data_ptr(),
                                        vs.data_ptr(), cap_sel, k_keep))
        kv = (sd.sd_seq_kv * (B * self.L))(*kvs)
        h0 = torch.stack([sdev.hidden(wl, b, self.dev) for b in range(B)])
        hid = h0.clone()
        ws = torch.empty(sd.sd_batch_workspace_bytes(self.dims, B), dtype=torch.uint8,
                         device=self.dev)
        d, dh = wl.d_model, wl.head_dim
        w_attn = 2 * (d * wl.qkv_out + wl.n_q_heads * dh * d)
        row = 2 * wl.n_kv_heads * dh * 2
        out = []
        for mode in modes:
            flags = self.mode_flags(mode)
            for i, c in enumerate(kv):
                c.n_full, c.n_sel = n, k_keep
            hid.copy_(h0)
            pos = [n] * B

            def steps(count):
                for _ in range(count):
                    sd.sd_decode_step_batch(self.dims, self.layers, kv, pos, hid, flags, ws)
                    for b in range(B):
                        pos[b] += 1

            steps(args.warmup)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            steps(args.steps)
            e1.record(self.stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            u = 1.0
            if flags & sd.SD_MLP_SPARSE:
                u = sum(float(m.float().mean()) for m in self.MASK) / self.L
            base = k_keep if flags & sd.SD_KV_SPARSE else n
            n_read = base + args.warmup + (args.steps - 1) / 2.0 + 1
            b_step = self.L * (w_attn + 2 * d * wl.d_ff * (1 + 2 * u) + B * row * n_read)
            out.append(dict(context=n, batch=B, mode=mode, us_per_step=ms * 1e3,
                            tokens_per_s=B / (ms * 1e-3), bytes_per_step=b_step,
                            gbs=b_step / ms / 1e6, hbm_frac=b_step / ms / 1e6 / HBM_PEAK_GBS,
                            union_fraction=u if flags & sd.SD_MLP_SPARSE else None))
        del keep, kv, ws, scores, idx, sws
        torch.cuda.empty_cache()
        return out

    def profile_cell(self, n, k_keep, mode):
        """Per-kernel event timing of the same steps (library profiler)."""
        torch, sd, args = self.torch, self.sd, self.args
        flags = self.mode_flags(mode)
        self.reset(n, k_keep, mode.startswith("catekv"))
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


# library profiler kind -> (rocprofv3 kernel name, source file)
KERNEL_SOURCES = {
    "qkv_rope_append": ("qkv_rope_append_kernel", "gemv.hip"),
    "attn_partial": ("attn_kernel", "attn.hip"),
    "attn_combine": ("attn_merge_kernel", "attn.hip"),
    "o_residual": ("o_residual_kernel", "gemv.hip"),
    "cats_gate_up": ("gate_kernel", "gemv.hip"),
    "cats_down": ("down_kernel", "down.hip"),
    "cats_reduce": ("mlp_reduce_kernel", "down.hip"),
}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


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
        if source_digest(KERNEL_SOURCES[kernel][1]) != rec["sha256"]:
            return None
        return rec["bytes_per_launch"]
    except Exception:
        return None


def pmc_summary(fetch_csv: str, write_csv: str, copy_bytes: int, out: str) -> None:
    """Per-kernel HBM bytes per dispatch from two rocprofv3 --pmc runs of this
    script (FETCH_SIZE, then WRITE_SIZE, in KiB), each scaled by what the same
    counter reads for the plain device copy of `copy_bytes` bytes that the runs
    start with (--pmc-copy-bytes).  The decode-step launches of a kernel are
    its most frequent grid size (calibration launches differ)."""
    import collections
    import csv
    import re

    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Correlation_Id"]))
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copy" in r["Kernel_Name"] and float(r["Counter_Value"]) * 1024 > copy_bytes / 4]
        if not copies:
            raise SystemExit(f"{path}: no copy-kernel dispatch of about {copy_bytes} bytes found")
        scale = copy_bytes / (sorted(copies)[len(copies) // 2] * 1024)
        per = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in rows:
            m = re.search(r"sd::(\w+)", r["Kernel_Name"])
            if m:
                per[m.group(1)][r["Grid_Size"]].append(float(r["Counter_Value"]) * 1024 * scale)
        return scale, per

    fs, fetch = load(fetch_csv, "FETCH_SIZE")
    ws, write = load(write_csv, "WRITE_SIZE")
    res = dict(about=("HBM bytes per dispatch of the decode-step kernels, from rocprofv3 --pmc "
                      "FETCH_SIZE and WRITE_SIZE, each scaled by the counter's reading for a "
                      f"plain {copy_bytes}-byte device copy"),
               fetch_scale=fs, write_scale=ws, kernels={})
    for kind, (rname, src) in KERNEL_SOURCES.items():
        if rname not in fetch or rname not in write:
            continue
        grid = max(fetch[rname], key=lambda g: len(fetch[rname][g]))
        f = fetch[rname][grid]
        w = write[rname].get(grid, [0.0])
        fb, wb = sum(f) / len(f), sum(w) / len(w)
        res["kernels"][kind] = dict(rocprof_name=rname, grid_size=int(grid), dispatches=len(f),
                                    fetch_bytes=round(fb), write_bytes=round(wb),
                                    bytes_per_launch=round(fb + wb), source=src,
                                    sha256=source_digest(src))
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


def cpu_baseline(bench, n, seconds):
    """The float64 oracle, timed as it stands on the host cores, on a bounded
    sample of the headline workload: the first layer of the stack (its own
    weights and 128K cache copied to the host), composed mode, repeated until
    `seconds` have passed; per-step time scaled to all layers."""
    import numpy as np
    import torch

    from oracle import cats as ocats, step as ostep

    wl = bench.wl
    W = {k: v.float().cpu().numpy() for k, v in bench.W[0].items()}
    reps_cap = 512
    shape = (wl.n_kv_heads, n + reps_cap, wl.head_dim)
    k = np.zeros(shape, np.float32)
    v = np.zeros(shape, np.float32)
    k[:, :n] = bench.K[0][:, :n].float().cpu().numpy()
    v[:, :n] = bench.V[0][:, :n].float().cpu().numpy()
    k_keep = int(math.floor(wl.keep_ratio * n))
    # the rows kept do not change the work; take the first k_keep rows
    ks = np.zeros((wl.n_kv_heads, k_keep + reps_cap, wl.head_dim), np.float32)
    vs = np.zeros_like(ks)
    ks[:, :k_keep] = k[:, :k_keep]
    vs[:, :k_keep] = v[:, :k_keep]
    h = bench.h0.cpu().numpy().astype(np.float64)
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
    per_step = per_layer * bench.L
    b = bench.step_bytes(k_keep + reps / 2.0 + 1, kept)
    cores, blas, single = 1, None, None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        info = threadpool_info()
        cores = max((p.get("num_threads", 1) for p in info), default=1)
        blas = ",".join(sorted({str(p.get("internal_api")) for p in info})) or None
        # the same oracle on one thread, a few more steps of the same layer
        r1, t1 = 0, time.perf_counter()
        with threadpool_limits(limits=1):
            while reps + r1 < reps_cap - 2 and (r1 == 0 or time.perf_counter() - t1 < seconds / 2):
                h = ostep.decode_layer(layer, h, n + reps + r1, kv_sparse=True, mlp_sparse=True,
                                       **dims)
                r1 += 1
        single = dict(value=b / ((time.perf_counter() - t1) / r1 * bench.L) / 1e9, steps=r1)
    except ImportError:
        pass
    return dict(value=b / per_step / 1e9, unit="GB/s", cores=int(cores), kind="oracle",
                ms_per_step=per_step * 1e3, blas=blas,
                affinity_cores=len(os.sched_getaffinity(0)),
                single_thread_gbs=None if single is None else round(single["value"], 4),
                single_thread_steps=None if single is None else single["steps"],
                sample=(f"float64 numpy oracle, layer 0 of the {bench.L}-layer stack at context "
                        f"{n}, composed mode (first {k_keep} rows as the gathered buffer, "
                        f"threshold at the median |a|), {reps} decode steps of that layer in "
                        f"{per_layer * reps:.1f} s; per-step time scaled x{bench.L} layers"))


def latency_gate(sweep):
    """The lookup table of a latency gate ([Cross] §3, "Dispatch and
    batching"): for each timed context and each decode length T, the mode
    with the least total time, T steps plus its one-time selection (KV
    modes).  Every timed mode is treated as admissible here: admissibility
    is a quality test that needs trained weights and real text."""
    out = []
    for n in sorted({c["context"] for c in sweep}):
        cells = [c for c in sweep if c["context"] == n]
        for T in GATE_HORIZONS:
            cost = {c["mode"]: T * c["ms_per_step"] + (c.get("select_ms") or 0.0) for c in cells}
            best = min(cost, key=cost.get)
            out.append(dict(context=n, horizon=T, best=best,
                            total_ms={k: round(v, 2) for k, v in cost.items()}))
    return out


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.pmc_copy_bytes, args.pmc_out)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported by this build "
              "(the sharded multi-GPU path is a design note only)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.pmc_copy_bytes:
        src = torch.ones(args.pmc_copy_bytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    bench = Bench(args)
    sweep = []
    sel_ms = {}
    for n in sorted(bench.contexts):
        secs, k_keep = bench.select(n)
        sel_ms[n] = secs * 1e3
        modes = [m for m in MODES if m in args.modes.split(",")]
        sel_r = bench.select_ragged(n) * 1e3 if bench.ragged else None
        for mode in modes:
            c = bench.cell(n, k_keep, mode)
            flags = bench.mode_flags(mode)
            c["select_ms"] = (sel_r if mode.startswith("catekv") else sel_ms[n]) \
                if flags & bench.sd.SD_KV_SPARSE else None
            sweep.append(c)
            print(f"# n={n:6d} {mode:5s} {c['us_per_step']:9.1f} us/step "
                  f"{c['gbs']:7.1f} GB/s ({100 * c['hbm_frac']:.1f}% of peak)"
                  + (f" keep {c['teal_keep']} (calibration off by <= {c['teal_calib_worst']}"
                     f" after {c['teal_calib_rounds']} Newton rounds)"
                     if "teal_keep" in c else ""), flush=True)
    n_head = max(bench.contexts)
    at_head = {c["mode"]: c for c in sweep if c["context"] == n_head}
    head = at_head.get("both") or next(iter(at_head.values()))
    dense, kv = at_head.get("dense"), at_head.get("kv")
    k_keep = int(math.floor(bench.wl.keep_ratio * n_head))
    bench.select(n_head)
    kern = bench.profile_cell(n_head, k_keep, head["mode"])
    dom = max((k for k in kern if "alg_bytes" in kern[k]), key=lambda k: kern[k]["total_ms"])
    dk = kern[dom]
    roof = dict(kernel=dom, bound="hbm", achieved=round(dk["gbs"], 1), peak=HBM_PEAK_GBS,
                unit="GB/s", frac=round(dk["frac"], 4), avg_us=round(dk["avg_us"], 2),
                alg_bytes_per_launch=dk["alg_bytes"], traffic=traffic_for(dom))
    payback = None
    if dense and kv and dense["ms_per_step"] > kv["ms_per_step"]:
        payback = sel_ms[n_head] / (dense["ms_per_step"] - kv["ms_per_step"])
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(bench, n_head, args.cpu_seconds)
    copy_gbs = bench.copy_ceiling()
    base = None
    if not args.no_attn_baselines:
        base = bench.attention_baselines(n_head)
        for k, v in base["paths"].items():
            print(f"# n={n_head:6d} {k:16s} {v['us_per_step']:9.1f} us/step, attention "
                  f"{v['attn_us_per_layer']:8.2f} us/layer = {100 * v['attn_frac_of_peak']:.1f}% of peak",
                  flush=True)
        print(f"# window speedups {base['window_speedup']} (byte bound {base['window_byte_bound']})",
              flush=True)
    batch = None
    if args.batches:
        cells = []
        for n in [int(c) for c in args.batch_contexts.split(",") if c]:
            for B in [int(b) for b in args.batches.split(",") if b]:
                for c in bench.batch_cells(n, B, ("dense", "kv", "cats", "both")):
                    cells.append(c)
                    print(f"# batch {B} n={n:6d} {c['mode']:5s} {c['us_per_step']:9.1f} us/step "
                          f"{c['tokens_per_s']:8.1f} tok/s {c['gbs']:7.1f} GB/s"
                          + (f" u_B {c['union_fraction']:.4f}" if c["union_fraction"] else ""),
                          flush=True)
        union = {}
        for B in sorted({c["batch"] for c in cells}):
            us = [c["union_fraction"] for c in cells if c["batch"] == B and c["union_fraction"]]
            u = sum(us) / len(us)
            n_star = bench.sd.sd_byte_crossover_batch(bench.dims, B, u, bench.wl.keep_ratio, 2.0,
                                                      2.0, bench.sd.SD_PROJ_CATS)
            union[str(B)] = dict(measured=round(u, 4), independent=round(1 - 0.5 ** B, 4),
                                 n_star_tokens=round(n_star, 1))
        batch = dict(cells=[{k: (round(v, 4) if isinstance(v, float) else v)
                             for k, v in c.items()} for c in cells], union=union)
    gate = latency_gate(sweep)
    for g in gate:
        print(f"# gate n={g['context']:6d} horizon {g['horizon']:5d}: {g['best']}", flush=True)
    line = dict(
        metric=METRIC, value=round(head["gbs"], 1), unit="GB/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(head["ms_per_step"], 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload=bench.wl.name if n_head == 131072 else f"8b-{bench.L}layer-both-ctx{n_head}",
                    layers=bench.L, context=n_head, mode="both", kv_keep=bench.wl.keep_ratio,
                    cats_sparsity=0.5, storage="bf16", accumulate="f32",
                    bytes_per_step=head["bytes_per_step"], hbm_frac=round(head["hbm_frac"], 4),
                    us_per_step=round(head["us_per_step"], 1),
                    us_per_step_blocks=head["us_per_step_blocks"],
                    select_ms_all_layers=round(sel_ms[n_head], 2),
                    select_payback_steps=None if payback is None else round(payback, 1)),
        roofline=roof, cpu_baseline=cpu,
        copy_ceiling_gbs=round(copy_gbs, 1),
        attention_baselines=base,
        latency_gate=gate,
        batch=batch,
        kernels={k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in e.items()}
                 for k, e in kern.items()},
        sweep=[{k: (round(v, 4) if isinstance(v, float) else v) for k, v in c.items()}
               for c in sweep],
    )
    s = json.dumps(line)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s + "\n")
    print(s, flush=True)


if __name__ == "__main__":
    main()
