"""CPU checks of bench.py's reporting: the last stdout line is one compact
JSON record that a log tail of a few KB holds whole, and the crossing and
latency-gate legs turn a sweep into the numbers of "Where Activation Sparsity
and KV-Cache Sparsity Cross in LLM Decoding" §4.3 and §3.3 through the
library's host calls."""

import json
import math
import types

import pytest

import bench
import synth

sd = pytest.importorskip("kv_cache_activation_amd", reason="libsd.so not built")
from oracle import byte_account as ba  # noqa: E402

CTX = [2048, 8192, 16384, 24576, 32768, 49152, 65536, 131072]


def _stack():
    wl = synth.STACK32_128K
    dims = sd.make_dims(wl.d_model, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff,
                        sd.SD_BF16, sd.SD_BF16)
    st = types.SimpleNamespace(sd=sd, dims=dims, L=32, wl=wl, contexts=CTX)
    st.mode_flags = lambda m: {"dense": 0, "kv": 4, "cats": 8, "both": 12}[m]
    return st


def _sweep(bw=5.5e12, cost=None):
    """Cells whose times follow bytes / bw + cost exactly, bytes from the
    oracle's account (CATS set, 50% keep, 10% KV keep)."""
    cost = cost or {"dense": 0.7e-3, "cats": 1.0e-3, "kv": 0.45e-3, "both": 0.8e-3}
    dm = ba.Dims(4096, 32, 8, 128, 14336)
    out = []
    for n in CTX:
        rec = ba.account(dm, 32, n, 0.5, 0.1, proj_set="cats")
        by = {"dense": rec.b_total, "cats": rec.b_total - rec.delta_p,
              "kv": rec.b_total - rec.delta_kv,
              "both": rec.b_total - rec.delta_p - rec.delta_kv}
        for m, b in by.items():
            us = (b / bw + cost[m]) * 1e6
            out.append(dict(context=n, mode=m, us=us, us_min=us, us_max=us, bytes=b,
                            gbs=b / us / 1e3, frac=b / us / 1e3 / 8000.0,
                            n_kept_mean=14336 * (0.5 if m in ("cats", "both") else 1.0),
                            select_ms=(3.0 if m in ("kv", "both") else None)))
    return out


def test_crossing_leg_recovers_the_linear_model_and_its_crossing():
    st = _stack()
    cost = {"dense": 0.7e-3, "cats": 1.0e-3, "kv": 0.45e-3, "both": 0.8e-3}
    cr = bench.crossing(st, _sweep(5.5e12, cost))
    assert abs(cr["bw_eff_gbs"] - 5500.0) <= 1e-6 * 5500
    for m, c in cost.items():
        assert abs(cr["cost_us"][m] - c * 1e6) <= 1e-6
    assert abs(cr["n_star_tokens"] - 31858.5) <= 1.0   # CATS up+down at (0.5, 0.1)
    # exact linear times: the interpolated crossing is the cost-aware prediction
    assert abs(cr["measured_cats_vs_kv_tokens"] - cr["n_lat_tokens"]) <= 1e-6 * cr["n_lat_tokens"]
    assert cr["n_lat_tokens"] < cr["n_star_tokens"]  # CATS carries the larger kernel cost


def test_latency_gate_leg_charges_the_selection():
    st = _stack()
    sweep = _sweep()
    gate = bench.latency_gate(st, sweep)
    assert len(gate) == len(CTX) * len(bench.GATE_HORIZONS)
    for g in gate:
        cells = [c for c in sweep if c["context"] == g["context"]]
        tot = {c["mode"]: g["horizon"] * c["us"] * 1e-3 + (c["select_ms"] or 0.0) for c in cells}
        assert g["best"] == min(tot, key=tot.get)


def test_headline_line_is_compact_json():
    st = _stack()
    sweep = _sweep()
    args = types.SimpleNamespace(steps=20, warmup=5, blocks=5, block_steps=50)
    head = dict(ms=2.6, bytes=1.19e10, gbs=4580.0, frac=0.5725)
    roof = dict(bound="hbm", achieved=5870.0, peak=8000.0, unit="GB/s", frac=0.7338,
                traffic=176900000, kernel="gate_kernel", avg_us=30.0,
                alg_bytes_per_launch=176000000.0)
    cpu = dict(value=2.1, unit="GB/s", cores=16, kind="oracle",
               sample="float64 numpy oracle, layer 0 of the stack at context 131072, composed "
                      "mode, 70 decode steps of that layer in 10.0 s, scaled x32 layers")
    cross = bench.crossing(st, sweep)
    line = bench.headline_line(args, st, head, roof, cpu, sweep, cross, 95.3)
    s = json.dumps(line, separators=(",", ":"))
    assert len(s) < 2500, len(s)
    back = json.loads(s)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in back, k
    assert back["dtype"] == "bf16" and back["config"]["workload"] == synth.STACK32_128K.name
    assert back["roofline"]["frac"] == 0.7338 and back["cpu_baseline"]["kind"] == "oracle"
    assert back["sweep"]["ctx"] == CTX and len(back["sweep"]["us"]["both"]) == len(CTX)
    assert not math.isnan(back["crossing"]["n_lat_k"])


def test_pmc_summary_maps_templated_kernels_and_scales(tmp_path):
    # two fake rocprofv3 counter CSVs: a 1 MiB copy kernel read as half its
    # bytes (FETCH) and as all of them (WRITE), then kernels whose full names
    # carry template arguments; each kind takes its own instances
    import csv
    import json

    import bench

    copy = 1 << 20
    rows = [("void at::copy_kernel(...)", 8192, copy / 2 / 1024, copy / 1024)]
    names = {
        "void sd::teal_kernel<unsigned short, false, 3, unsigned short>(sd::TealArgs)": 135168,
        "void sd::teal_kernel<unsigned short, false, 1, float>(sd::TealArgs)": 131072,
        "void sd::teal_kernel<unsigned short, true, 2, float>(sd::TealArgs)": 143360,
        "void sd::bmma_kernel<8, false, 1, 16>(sd::BmmaArgs)": 131072,
        "void sd::bmma_kernel<8, false, 1, 32>(sd::BmmaArgs)": 229376,
        "void sd::teal_kernel<unsigned short, false, 5, float>(sd::TealArgs)": 131072,
        "void sd::teal_kernel<unsigned short, false, 4, float>(sd::TealArgs)": 131072,
        "void sd::down_kernel<unsigned short, 1>(sd::DownArgs)": 131072,
    }
    for i, (n, g) in enumerate(names.items()):
        for _ in range(3):
            rows.append((n, g, 100.0 * (i + 1), 10.0 * (i + 1)))

    def write(path, counter, col):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, ["Correlation_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                   "Counter_Value"])
            w.writeheader()
            for cid, r in enumerate(rows):
                w.writerow(dict(Correlation_Id=cid, Kernel_Name=r[0], Grid_Size=r[1],
                                Counter_Name=counter, Counter_Value=r[col]))

    fc, wc, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    write(fc, "FETCH_SIZE", 2)
    write(wc, "WRITE_SIZE", 3)
    bench.pmc_summary(str(fc), str(wc), copy, str(out))
    res = json.load(open(out))
    assert abs(res["fetch_scale"] - 2.0) < 1e-9 and abs(res["write_scale"] - 1.0) < 1e-9
    k = res["kernels"]
    # index of each kind's row in `names` (+1) sets its counter values
    want = {"teal_qkv": 1, "teal_o": 2, "teal_gate_up": 3, "batch_o": 4, "batch_down": 5,
            "cats_down": 6, "teal_down": 7}
    for kind, i in want.items():
        assert k[kind]["fetch_bytes"] == round(100.0 * i * 1024 * 2.0), kind
        assert k[kind]["write_bytes"] == round(10.0 * i * 1024), kind
        assert k[kind]["dispatches"] == 3
    assert "batch_qkv" not in k and "qkv_rope_append" not in k
