"""Cases that compare the library's host-side byte account, sweep fit,
crossing and latency gate with the oracle's (same arguments on both sides).
Used by the CPU ABI tests and by the GPU suite, so that the account is
checked on the machine whose measurements it explains."""

import math

from oracle import byte_account as ba

DIMS8B = dict(d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, d_ff=14336)
PROJ = [("all7", 0), ("ffn", 1), ("cats", 2)]
POINTS = [(2048, 0.5, 0.3, 2, 0.0), (131072, 0.5, 0.3, 2, 1.05e9), (32768, 0.5, 0.1, 0.5, 0.0),
          (65536, 0.3, 1.0, 2, 0.0), (8192, 0.0, 0.0, 1, 0.0)]
LATENCY = [None, (5.6e12, 0.9e-3, 0.3e-3), (1.57e12, 2.0e-3, 0.0), (8e12, 0.0, 0.0)]
FIELDS = ("b_attn", "b_mlp", "b_kv", "b_total", "delta_p", "delta_kv", "bound_p", "bound_kv",
          "bound_both", "n_star", "n_star_budget", "gap_per_k", "n_lat")


def _same(a, b, rel=1e-12):
    if math.isnan(b):
        return math.isnan(a)
    if math.isinf(b):
        return a == b
    return abs(a - b) <= rel * abs(b)


def check_account(sd, dims, proj, code, point, latency):
    n, r_p, r_kv, s_w, lm = point
    kw = {}
    if latency is not None:
        kw = dict(bw_eff=latency[0], c_p=latency[1], c_kv=latency[2])
    want = ba.account(ba.Dims(**DIMS8B), 32, n, r_p, r_kv, s_w=s_w, s_kv=2, proj_set=proj,
                      fixed_bytes=lm, **kw)
    got = sd.sd_byte_account(dims, 32, n, r_p, r_kv, s_w, 2.0, code, lm, latency=latency)
    for f in FIELDS:
        assert _same(getattr(got, f), getattr(want, f)), (f, getattr(got, f), getattr(want, f))


BATCH = [(4, 0.92, 0.3, 2), (8, 0.985, 0.1, 2), (4, 0.9375, 0.2, 0.5), (1, 0.5, 0.3, 2)]


def check_batched(sd, dims, proj, code, case):
    batch, u_b, r_kv, s_w = case
    want = ba.crossover_batched(ba.Dims(**DIMS8B), batch, u_b, r_kv, s_w, 2.0, proj)
    got = sd.sd_byte_crossover_batch(dims, batch, u_b, r_kv, s_w, 2.0, code)
    assert _same(got, want)
    assert math.isinf(sd.sd_byte_crossover_batch(dims, batch, u_b, 1.0, s_w, 2.0, code))


def sweep(seed):
    """A measured-looking sweep: the account's bytes of the 8B-class stack
    (CATS set, 50% / 10% keep) at eight contexts, times = bytes / bw + cost
    with seeded noise (so nothing is exactly linear)."""
    import numpy as np
    r = np.random.default_rng(seed)
    ctx = [2048, 8192, 16384, 24576, 32768, 49152, 65536, 131072]
    dm = ba.Dims(**DIMS8B)
    bw = 4.5e12 + 1e12 * r.random()
    rows = {"dense": [], "p": [], "kv": [], "both": []}
    for n in ctx:
        rec = ba.account(dm, 32, n, 0.5, 0.1, proj_set="cats")
        rows["dense"].append(rec.b_total)
        rows["p"].append(rec.b_total - rec.delta_p)
        rows["kv"].append(rec.b_total - rec.delta_kv)
        rows["both"].append(rec.b_total - rec.delta_p - rec.delta_kv)
    cost = {"dense": 0.6e-3, "p": 0.8e-3 + 0.4e-3 * r.random(), "kv": 0.3e-3, "both": 0.9e-3}
    t = {k: [cost[k] + b / bw + 2e-5 * r.standard_normal() for b in v] for k, v in rows.items()}
    return ctx, rows, t


def check_sweep(sd, seed):
    ctx, rows, t = sweep(seed)
    modes = ["p", "kv", "both"]
    bw, c = sd.sd_latency_fit(rows["dense"], t["dense"], [rows[m] for m in modes],
                              [t[m] for m in modes])
    bw_o = ba.effective_bandwidth(rows["dense"], t["dense"])
    assert _same(bw, bw_o, 1e-10)
    for m, cm in zip(modes, c):
        assert abs(cm - ba.kernel_cost(rows[m], t[m], bw_o)) <= 1e-12
    for a, b in (("p", "kv"), ("dense", "kv"), ("p", "both"), ("dense", "p")):
        assert _same(sd.sd_latency_crossing(ctx, t[a], t[b]),
                     ba.measured_crossing(ctx, t[a], t[b]), 1e-12)


def check_gate(sd, seed):
    import numpy as np
    r = np.random.default_rng(seed)
    n = 6
    t_step = list(1e-3 * (1 + r.random(n)))
    t_once = [0.0 if i % 2 == 0 else 1e-2 * r.random() for i in range(n)]
    t_step[3] = t_step[1]  # a tie candidate
    t_once[3] = t_once[1]
    for horizon in (0, 1, 16, 256, 4096, 1 << 20):
        for adm in (None, [1, 0, 1, 1, 0, 1], [0] * n):
            assert sd.sd_latency_gate(t_step, t_once, horizon, adm) == \
                ba.latency_gate(t_step, t_once, horizon, adm)
