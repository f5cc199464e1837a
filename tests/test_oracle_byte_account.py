"""Pins of the oracle's byte account against the numbers the subject page prints.

Fixture: tests/golden/byte_account_pins.json (each entry cites its section of
"Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding").
"""

import json
import math
import os

import pytest

from oracle import byte_account as ba

HERE = os.path.dirname(__file__)
GOLD = json.load(open(os.path.join(HERE, "golden", "byte_account_pins.json")))
DIMS = ba.Dims(**{k: GOLD["dims"][k] for k in ("d_model", "n_q_heads", "n_kv_heads",
                                                 "head_dim", "d_ff")})
L = GOLD["dims"]["n_layers"]
LM = GOLD["lm_head_bytes"]


def _pin(pid):
    return next(p for p in GOLD["pins"] if p["id"] == pid)


@pytest.mark.parametrize("pid", ["n_star_nominal", "n_star_budget_1.0"])
def test_crossover_printed(pid):
    p = _pin(pid)
    n = ba.crossover(DIMS, p["r_p"], p["r_kv"], 2, 2, p["proj_set"]) / ba.K_TOKENS
    assert abs(n - p["printed"]) <= p["abs_tol"], (pid, n)


def test_batched_crossover_printed():
    p = _pin("batched_n4")
    n = ba.crossover_batched(DIMS, p["batch"], p["u_b"], p["r_kv"], 2, 2) / ba.K_TOKENS
    assert abs(n - p["printed"]) <= p["abs_tol"]
    # §3.3: at most n*/B (u_B >= r_P), and "far below" it at 92% coverage
    assert n < ba.crossover(DIMS, 0.5, p["r_kv"], 2, 2) / ba.K_TOKENS / p["batch"]


def test_precision_scaling_printed():
    p = _pin("precision_4bit")
    a = ba.crossover(DIMS, p["r_p"], p["r_kv"], p["s_w_a"], 2)
    b = ba.crossover(DIMS, p["r_p"], p["r_kv"], p["s_w_b"], 2)
    assert abs(a / b - p["printed"]) <= p["abs_tol"]


def test_kv_bound_printed_needs_lm_head():
    p = _pin("kv_bound_128k_30")
    with_lm = ba.account(DIMS, L, p["n"], 1.0, p["r_kv"], fixed_bytes=LM).bound_kv
    without = ba.account(DIMS, L, p["n"], 1.0, p["r_kv"]).bound_kv
    assert abs(with_lm - p["printed"]) <= p["abs_tol"], with_lm
    assert abs(without - p["printed"]) > p["abs_tol"]  # the reading is forced


@pytest.mark.parametrize("pid", ["latency_shift_a100", "latency_shift_a6000"])
def test_latency_shift_printed(pid):
    p = _pin(pid)
    n_star = 100_000.0
    n_lat = ba.latency_crossing(n_star, p["dc_ms"], 0.0, p["s_ms_per_k"])
    assert abs((n_star - n_lat) / ba.K_TOKENS - p["printed"]) <= p["abs_tol"]


@pytest.mark.parametrize("row", GOLD["measured_below_bound"], ids=lambda r: r["cite"][:30])
def test_measured_speedups_sit_below_bounds(row):
    rec = ba.account(DIMS, L, row["n"], row["r_p"], row["r_kv"], fixed_bytes=LM)
    bound = {"p": rec.bound_p, "kv": rec.bound_kv, "both": rec.bound_both}[row["branch"]]
    for m in row["measured"]:
        assert m < bound, (m, bound)


def test_within_of_bound():
    row = GOLD["within_of_bound"][0]
    rec = ba.account(DIMS, L, row["n"], row["r_p"], row["r_kv"], fixed_bytes=LM)
    assert rec.bound_kv * (1 - row["within"]) <= row["measured"] <= rec.bound_kv


def test_savings_equal_at_crossover():
    for r_p, r_kv in [(0.5, 0.3), (0.5, 0.1), (0.3, 0.6)]:
        for ps in ba.PROJ_SETS:
            n = ba.crossover(DIMS, r_p, r_kv, 2, 2, ps)
            dp = ba.delta_p(DIMS, L, r_p, 2, ps)
            dk = ba.delta_kv(DIMS, L, n, r_kv, 2)
            assert abs(dp - dk) <= 1e-9 * dp


def test_fixed_budget_matches_general_form():
    # §3.3: substituting r_KV = b/n into the general crossover gives b + P(1-r_P)/(2 h_kv d_h)
    b = 2048.0
    n = ba.crossover_fixed_budget(DIMS, b, 0.5, 2, 2)
    assert n > b
    n_general = ba.crossover(DIMS, 0.5, b / n, 2, 2)
    assert abs(n_general - n) <= 1e-9 * n


def test_bounds_move_with_context_as_stated():
    # §3.3: the projection bound falls with n, the KV bound rises, both together is largest
    ns = [2048, 8192, 32768, 65536, 131072]
    recs = [ba.account(DIMS, L, n, 0.5, 0.3) for n in ns]
    assert all(a.bound_p > b.bound_p for a, b in zip(recs, recs[1:]))
    assert all(a.bound_kv < b.bound_kv for a, b in zip(recs, recs[1:]))
    assert all(r.bound_both > max(r.bound_p, r.bound_kv) for r in recs)


def test_keep_ratio_one_disables_branch():
    rec = ba.account(DIMS, L, 32768, 1.0, 1.0)
    assert rec.delta_p == 0 and rec.delta_kv == 0 and rec.bound_both == 1.0


def test_projection_sets_nest():
    assert ba.sparse_params(DIMS, "cats") < ba.sparse_params(DIMS, "ffn") < ba.sparse_params(DIMS, "all7")
    # up and down are two thirds of the feed-forward weights
    assert 3 * ba.sparse_params(DIMS, "cats") == 2 * ba.sparse_params(DIMS, "ffn")


def test_step_bytes_dense_equals_account_total():
    # the executed-traffic count reduces to the account's B_total(n+1) plus the
    # appended row when nothing is sparse and no gathered buffer exists
    n = 8192
    got = ba.step_bytes(DIMS, L, n + 1, DIMS.d_ff, 2, 2, has_sel=False)
    want = ba.b_total(DIMS, L, n + 1, 2, 2) + L * ba.b_kv(DIMS, 1, 2)
    assert got == want


def test_gap_growth_printed_a100():
    # s of §4.3 from the byte account and the A100's effective bandwidth
    # (78% of its peak, the split-K share that §4.4 prints)
    p = _pin("gap_growth_a100")
    s = ba.gap_growth_per_k(DIMS, L, p["r_kv"], 2, p["peak_bytes_per_s"] * p["frac_of_peak"])
    assert abs(s * 1e3 - p["printed"]) <= p["abs_tol"], s


@pytest.mark.parametrize("r_kv,bw,n", [(0.3, 1.6e12, 4096), (0.1, 5.6e12, 100000), (0.0, 8e12, 0)])
def test_gap_growth_is_the_kv_saving_of_1k_more_tokens_over_bandwidth(r_kv, bw, n):
    # s is how much the KV branch's skipped bytes grow over 1024 tokens, in time
    s = ba.gap_growth_per_k(DIMS, L, r_kv, 2, bw)
    grow = ba.delta_kv(DIMS, L, n + ba.K_TOKENS, r_kv, 2) - ba.delta_kv(DIMS, L, n, r_kv, 2)
    assert abs(s * bw - grow) <= 1e-9 * grow


def _linear_sweep(bw, c):
    """Times of dense, CATS-branch and KV-branch steps that are exactly
    c_X + bytes_X / bw, with bytes from the account (CATS set, 50% / 10%)."""
    ctx = [2048, 8192, 16384, 32768, 65536, 131072]
    bd, bp, bk = [], [], []
    for n in ctx:
        rec = ba.account(DIMS, L, n, 0.5, 0.1, proj_set="cats")
        bd.append(rec.b_total)
        bp.append(rec.b_total - rec.delta_p)
        bk.append(rec.b_total - rec.delta_kv)
    t = {k: [c[k] + b / bw for b in bs] for k, bs in (("dense", bd), ("p", bp), ("kv", bk))}
    return ctx, bd, bp, bk, t


def test_sweep_fit_recovers_an_exactly_linear_latency_model():
    bw = 5.0e12
    c = {"dense": 0.5e-3, "p": 0.9e-3, "kv": 0.3e-3}
    ctx, bd, bp, bk, t = _linear_sweep(bw, c)
    got_bw = ba.effective_bandwidth(bd, t["dense"])
    assert abs(got_bw - bw) <= 1e-9 * bw
    for k, b in (("dense", bd), ("p", bp), ("kv", bk)):
        assert abs(ba.kernel_cost(b, t[k], got_bw) - c[k]) <= 1e-12


def test_measured_crossing_of_linear_curves_is_the_cost_aware_prediction():
    # t_P - t_KV is linear in n when both follow bytes/bw + c, so the
    # interpolated crossing is exact and equals n_lat = n* - (c_P - c_KV)/s
    bw = 5.0e12
    for c_p, c_kv in [(0.9e-3, 0.3e-3), (0.3e-3, 0.3e-3), (0.2e-3, 0.25e-3)]:
        ctx, bd, bp, bk, t = _linear_sweep(bw, {"dense": 0.0, "p": c_p, "kv": c_kv})
        rec = ba.account(DIMS, L, 32768, 0.5, 0.1, proj_set="cats", bw_eff=bw, c_p=c_p, c_kv=c_kv)
        n_cross = ba.measured_crossing(ctx, t["p"], t["kv"])
        assert ctx[0] < rec.n_lat < ctx[-1]
        assert abs(n_cross - rec.n_lat) <= 1e-6 * rec.n_lat
        if c_p == c_kv:  # equal kernel costs: the latency crossing is the byte crossover
            assert abs(rec.n_lat - rec.n_star) <= 1e-9 * rec.n_star


def test_measured_crossing_hand_cases():
    assert ba.measured_crossing([1, 2, 3], [0, 1, 5], [1, 2, 2]) == 2.25
    assert ba.measured_crossing([1, 2, 3], [0, 2, 5], [1, 2, 2]) == 2.0  # an exact tie
    assert math.isnan(ba.measured_crossing([1, 2, 3], [0, 1, 1], [1, 2, 2]))
    # the first sign change counts
    assert ba.measured_crossing([10, 20, 30, 40], [0, 4, 0, 4], [2, 2, 2, 2]) == 15.0


def test_latency_gate_hand_cases():
    t_step, t_once = [3.0, 2.0, 1.5], [0.0, 10.0, 40.0]
    # totals at horizon 1: 3, 12, 41.5; at 20: 60, 50, 70; at 100: 300, 210, 190
    assert [ba.latency_gate(t_step, t_once, h) for h in (1, 20, 100)] == [0, 1, 2]
    assert ba.latency_gate([1.0, 1.0], [0.0, 0.0], 7) == 0  # ties to the lower index
    assert ba.latency_gate(t_step, t_once, 100, admissible=[1, 1, 0]) == 1
    assert ba.latency_gate(t_step, t_once, 100, admissible=[0, 0, 0]) == -1


def test_record_budget_crossover_and_latency_fields():
    rec = ba.account(DIMS, L, 65536, 0.5, 0.1, proj_set="cats")
    assert math.isnan(rec.gap_per_k) and math.isnan(rec.n_lat)
    b = 0.1 * 65536
    assert rec.n_star_budget == ba.crossover_fixed_budget(DIMS, b, 0.5, 2, 2, "cats")
    # at that crossing the fixed-budget method's keep ratio b / n* gives the general n*
    n_general = ba.crossover(DIMS, 0.5, b / rec.n_star_budget, 2, 2, "cats")
    assert abs(n_general - rec.n_star_budget) <= 1e-9 * n_general
