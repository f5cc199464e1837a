"""CPU-side checks of the C ABI: the library loads, exports every symbol that
include/sd.h declares, rejects bad arguments before touching the GPU, and its
host-only byte account agrees with the oracle's independent one."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sd.h")

sd = pytest.importorskip("kv_cache_activation_amd", reason="libsd.so not built")

import account_cases  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sd_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(sd.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(sd.EXPORTS)


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(sd.sd_dims) == 36
    assert ctypes.sizeof(sd.sd_layer) == 240
    assert ctypes.sizeof(sd.sd_byte_record) == 104
    assert ctypes.sizeof(sd.sd_latency_model) == 24
    assert ctypes.sizeof(sd.sd_seq_kv) == 48


def test_struct_layout_matches_the_c_compiler(tmp_path):
    # every field offset of the ctypes mirrors equals the C compiler's offsetof
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("no C compiler")
    structs = {"sd_dims": sd.sd_dims, "sd_layer": sd.sd_layer, "sd_byte_record": sd.sd_byte_record,
               "sd_seq_kv": sd.sd_seq_kv, "sd_latency_model": sd.sd_latency_model}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "sd.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'  printf("{name} %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-I", inc, str(src), "-o", str(tmp_path / "layout")], check=True)
    out = subprocess.run([str(tmp_path / "layout")], capture_output=True, text=True,
                         check=True).stdout.split("\n")
    got = dict(l.split() for l in out if l)
    for name, cls in structs.items():
        assert int(got[name]) == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert int(got[f"{name}.{f}"]) == getattr(cls, f).offset, (name, f)


DIMS8B = dict(d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, d_ff=14336)


def _dims(**over):
    kw = dict(DIMS8B, w_dtype=sd.SD_BF16, kv_dtype=sd.SD_BF16)
    kw.update(over)
    return sd.make_dims(**kw)


def test_status_strings():
    assert sd.sd_status_string(sd.SD_OK) == "ok"
    assert "workspace" in sd.sd_status_string(sd.SD_ENOSPC)


def test_workspace_bytes_grows_with_rows_and_window():
    a = sd.sd_workspace_bytes(_dims(), 0, 0)
    b = sd.sd_workspace_bytes(_dims(), 131072, 32)
    assert 0 < a < b
    assert sd.sd_workspace_bytes(_dims(head_dim=96), 1024, 32) == 0  # unsupported dims


FAKE = 1 << 20  # aligned address; never dereferenced because validation fails first


class _FakeWs:
    def __init__(self, nbytes):
        self.n = nbytes

    def data_ptr(self):
        return FAKE

    def numel(self):
        return self.n

    def element_size(self):
        return 1


@pytest.mark.parametrize("case,status", [
    (dict(n_ctx=0), sd.SD_EINVAL),
    (dict(n_ctx=10, cap=5), sd.SD_EINVAL),
    (dict(q=FAKE + 4), sd.SD_EINVAL),
    (dict(q=None), sd.SD_EINVAL),
    (dict(ws_bytes=16), sd.SD_ENOSPC),
    (dict(n_splits=100000), sd.SD_ENOSPC),
    (dict(dims=dict(head_dim=96)), sd.SD_EUNSUPPORTED),
    (dict(dims=dict(n_q_heads=24, n_kv_heads=8)), sd.SD_EUNSUPPORTED),
    (dict(dims=dict(n_q_heads=30)), sd.SD_EINVAL),
    (dict(dims=dict(d_model=4100)), sd.SD_EUNSUPPORTED),
    (dict(dims=dict(w_dtype=7)), sd.SD_EUNSUPPORTED),
])
def test_decode_attn_rejects_before_launch(case, status):
    dims = _dims(**case.get("dims", {}))
    ws = _FakeWs(case.get("ws_bytes", 1 << 30))
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_attn(dims, case.get("q", FAKE), FAKE, FAKE, case.get("cap", 100),
                          case.get("n_ctx", 50), 0.1, case.get("n_splits", 0), FAKE, None, ws, 0)
    assert e.value.status == status
    assert sd.sd_last_error()


@pytest.mark.parametrize("case,status", [
    (dict(w=0), sd.SD_EINVAL),
    (dict(w=200), sd.SD_EINVAL),
    (dict(k_keep=20, n_sink=4, w=32), sd.SD_EINVAL),
    (dict(cap_sel=10), sd.SD_ENOSPC),
    (dict(n=200), sd.SD_EINVAL),
])
def test_select_kv_rejects_before_launch(case, status):
    a = dict(n=100, w=8, n_sink=4, k_keep=40, cap_sel=64)
    a.update(case)
    with pytest.raises(sd.SdError) as e:
        sd.sd_select_kv(_dims(), FAKE, FAKE, 128, a["n"], FAKE, a["w"], a["n_sink"], a["k_keep"],
                        FAKE, FAKE, FAKE, FAKE, a["cap_sel"], 0, _FakeWs(1 << 30), 0)
    assert e.value.status == status


def test_decode_step_rejects_full_cache_and_missing_buffer():
    lay = sd.sd_layer(*([FAKE] * 7), 0.1, 0, FAKE, FAKE, 64, 64, None, None, 0, 0, None)
    layers = (sd.sd_layer * 1)(lay)
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step(_dims(), layers, 64, FAKE, 0, _FakeWs(1 << 30), 0)
    assert e.value.status == sd.SD_ENOSPC
    layers[0].n_full = 10
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step(_dims(), layers, 10, FAKE, sd.SD_KV_SPARSE, _FakeWs(1 << 30), 0)
    assert e.value.status == sd.SD_EINVAL
    assert layers[0].n_full == 10  # untouched on failure


def test_sparse_mlp_rejects_nan_threshold():
    with pytest.raises(sd.SdError) as e:
        sd.sd_sparse_mlp(_dims(), FAKE, None, FAKE, FAKE, FAKE, float("nan"), FAKE, FAKE, FAKE,
                         FAKE, 0, _FakeWs(1 << 30), 0)
    assert e.value.status == sd.SD_EINVAL


@pytest.mark.parametrize("proj,code", account_cases.PROJ)
@pytest.mark.parametrize("point", account_cases.POINTS)
@pytest.mark.parametrize("latency", account_cases.LATENCY)
def test_byte_account_matches_oracle(proj, code, point, latency):
    account_cases.check_account(sd, _dims(), proj, code, point, latency)


@pytest.mark.parametrize("proj,code", account_cases.PROJ)
@pytest.mark.parametrize("case", account_cases.BATCH)
def test_batched_crossover_matches_oracle(proj, code, case):
    account_cases.check_batched(sd, _dims(), proj, code, case)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_latency_fit_and_crossing_match_oracle(seed):
    account_cases.check_sweep(sd, seed)


@pytest.mark.parametrize("seed", [0, 1])
def test_latency_gate_matches_oracle(seed):
    account_cases.check_gate(sd, seed)


def test_latency_helpers_reject_bad_input():
    with pytest.raises(sd.SdError):  # one point gives no slope
        sd.sd_latency_fit([1.0], [1.0], [], [])
    with pytest.raises(sd.SdError):  # time falling with bytes
        sd.sd_latency_fit([1.0, 2.0], [2.0, 1.0], [], [])
    with pytest.raises(sd.SdError):  # contexts must ascend
        sd.sd_latency_crossing([2.0, 1.0], [0.0, 1.0], [1.0, 0.0])
    with pytest.raises(sd.SdError):
        sd.sd_latency_gate([1.0, -1.0], [0.0, 0.0], 10)
    with pytest.raises(sd.SdError):  # a latency model needs a positive bandwidth
        sd.sd_byte_account(_dims(), 32, 1024, 0.5, 0.3, 2, 2, sd.SD_PROJ_ALL7,
                           latency=(0.0, 1e-3, 0.0))


def test_byte_account_rejects_bad_ratio():
    with pytest.raises(sd.SdError):
        sd.sd_byte_account(_dims(), 32, 1024, 1.5, 0.3, 2, 2, sd.SD_PROJ_ALL7)


def test_window_and_baseline_reject_before_launch():
    ws = _FakeWs(1 << 30)
    with pytest.raises(sd.SdError) as e:   # sinks beyond the window
        sd.sd_decode_attn_window(_dims(), FAKE, FAKE, FAKE, 100, 50, 10, 5, 0.1, 0, FAKE, None, ws, 0)
    assert e.value.status == sd.SD_EINVAL
    with pytest.raises(sd.SdError) as e:   # more rows than the cache holds
        sd.sd_decode_attn_window(_dims(), FAKE, FAKE, FAKE, 100, 101, 4, 20, 0.1, 0, FAKE, None, ws, 0)
    assert e.value.status == sd.SD_EINVAL
    with pytest.raises(sd.SdError) as e:   # not a comparison path
        sd.sd_decode_attn_baseline(_dims(), FAKE, FAKE, FAKE, 100, 50, 0.1, 0, FAKE, None, ws, 0)
    assert e.value.status == sd.SD_EINVAL
    small = _FakeWs(sd.sd_workspace_bytes(_dims(), 0, 0))  # no room for the score rows
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_attn_baseline(_dims(), FAKE, FAKE, FAKE, 100000, 50, 0.1, sd.SD_ATTN_MASKED,
                                   FAKE, None, small, 0)
    assert e.value.status == sd.SD_ENOSPC


@pytest.mark.parametrize("case,status", [
    (dict(d_in=12), sd.SD_EINVAL),
    (dict(d_out=0), sd.SD_EINVAL),
    (dict(d_in=40000), sd.SD_EUNSUPPORTED),
    (dict(x=FAKE + 4), sd.SD_EINVAL),
    (dict(t=float("nan")), sd.SD_EINVAL),
    (dict(flags=1), sd.SD_EINVAL),
    (dict(w2=FAKE, y2=None), sd.SD_EINVAL),
    (dict(d_in=32768, d_out=32768, w2=FAKE, y2=FAKE), sd.SD_ENOSPC),
    (dict(ws_bytes=64), sd.SD_ENOSPC),
])
def test_teal_gemv_rejects_before_launch(case, status):
    a = dict(x=FAKE, d_in=4096, d_out=4096, t=0.5, w2=None, y2=None, flags=0, ws_bytes=1 << 30)
    a.update(case)
    with pytest.raises(sd.SdError) as e:
        sd.sd_teal_gemv(_dims(), a["x"], a["d_in"], None, a["t"], FAKE, a["w2"], a["d_out"], FAKE,
                        a["y2"], a["flags"], None, None, _FakeWs(a["ws_bytes"]), 0)
    assert e.value.status == status


def test_decode_step_teal_needs_block_weights_and_no_cats():
    L = (sd.sd_layer * 1)()
    l = L[0]
    for f in ("attn_norm", "mlp_norm", "w_down_t", "k_full", "v_full"):
        setattr(l, f, FAKE)
    l.cap_full, l.n_full = 100, 10
    ws = _FakeWs(1 << 30)
    with pytest.raises(sd.SdError) as e:  # no column-block weights
        sd.sd_decode_step(_dims(), L, 10, FAKE, sd.SD_PROJ_TEAL, ws, 0)
    assert e.value.status == sd.SD_EINVAL and "column-block" in sd.sd_last_error()
    for f in ("w_qkv_t", "w_o_t", "w_gate_t", "w_up_t"):
        setattr(l, f, FAKE)
    with pytest.raises(sd.SdError) as e:  # excludes CATS
        sd.sd_decode_step(_dims(), L, 10, FAKE, sd.SD_PROJ_TEAL | sd.SD_MLP_SPARSE, ws, 0)
    assert e.value.status == sd.SD_EINVAL
    l.teal_t[2] = float("nan")
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step(_dims(), L, 10, FAKE, sd.SD_PROJ_TEAL, ws, 0)
    assert e.value.status == sd.SD_EINVAL and "NaN" in sd.sd_last_error()
    l.teal_t[2] = 0.1
    l.teal_masks_out = FAKE + 8
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step(_dims(), L, 10, FAKE, sd.SD_PROJ_TEAL, ws, 0)
    assert e.value.status == sd.SD_EINVAL


@pytest.mark.parametrize("mode", [sd.SD_KV_SPARSE | sd.SD_KV_WINDOW,
                                  sd.SD_ATTN_MASKED | sd.SD_ATTN_FUSED,
                                  sd.SD_KV_SPARSE | sd.SD_ATTN_FUSED, 1 << 9])
def test_decode_step_rejects_conflicting_modes(mode):
    lay = sd.sd_layer(*([FAKE] * 7), 0.1, 0, FAKE, FAKE, 64, 10, FAKE, FAKE, 64, 10, None, 8, 4)
    layers = (sd.sd_layer * 1)(lay)
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step(_dims(), layers, 10, FAKE, mode, _FakeWs(1 << 30), 0)
    assert e.value.status == sd.SD_EINVAL
    assert layers[0].n_full == 10


@pytest.mark.parametrize("case,status", [
    (dict(k=[40, 40, 40, 10, 40, 40, 40, 40]), sd.SD_EINVAL),   # one head below n_sink + w
    (dict(stride=30), sd.SD_EINVAL),                            # stride below the largest count
    (dict(cap_sel=39), sd.SD_ENOSPC),
    (dict(w=0), sd.SD_EINVAL),
    (dict(dims=dict(n_q_heads=64, n_kv_heads=64, d_model=8192)), sd.SD_EUNSUPPORTED),
])
def test_select_kv_ragged_rejects_before_launch(case, status):
    a = dict(n=100, w=8, n_sink=4, k=[12, 40, 100, 150, 12, 12, 40, 20], stride=100, cap_sel=100)
    a.update(case)
    dims = _dims(**case.get("dims", {}))
    k = a["k"] if dims.n_kv_heads == 8 else [40] * dims.n_kv_heads
    if case.get("cap_sel"):
        k = [40] * 8
        a["stride"] = 40
    with pytest.raises(sd.SdError) as e:
        sd.sd_select_kv_ragged(dims, FAKE, FAKE, 128, a["n"], FAKE, a["w"], a["n_sink"], k,
                               FAKE, FAKE, a["stride"], FAKE, FAKE, a["cap_sel"], 0,
                               _FakeWs(1 << 30), 0)
    assert e.value.status == status


@pytest.mark.parametrize("case,status", [
    (dict(lens=[10, 0, 10, 10, 10, 10, 10, 10]), sd.SD_EINVAL),
    (dict(lens=[10, 10, 10, 10, 10, 10, 10, 101]), sd.SD_EINVAL),
    (dict(n_splits=100000), sd.SD_ENOSPC),
    (dict(q=None), sd.SD_EINVAL),
])
def test_decode_attn_ragged_rejects_before_launch(case, status):
    lens = case.get("lens", [10, 20, 30, 40, 50, 60, 70, 80])
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_attn_ragged(_dims(), case.get("q", FAKE), FAKE, FAKE, 100, lens, 0.1,
                                 case.get("n_splits", 0), FAKE, None, _FakeWs(1 << 30), 0)
    assert e.value.status == status


def test_decode_step_ragged_checks_every_head_and_advances_each():
    L = (sd.sd_layer * 1)()
    l = L[0]
    for f in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down_t", "k_full",
              "v_full", "k_sel", "v_sel"):
        setattr(l, f, FAKE)
    l.cap_full, l.n_full, l.cap_sel = 100, 10, 50
    heads = (ctypes.c_int32 * 8)(5, 6, 7, 8, 9, 50, 11, 12)   # head 5 has no free row
    l.n_sel_heads = heads
    ws = _FakeWs(1 << 30)
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step(_dims(), L, 10, FAKE, sd.SD_KV_SPARSE, ws, 0)
    assert e.value.status == sd.SD_ENOSPC and "head 5" in sd.sd_last_error()
    heads[5] = 10
    with pytest.raises(sd.SdError) as e:   # ragged budgets exclude the window
        sd.sd_decode_step(_dims(), L, 10, FAKE, sd.SD_KV_WINDOW, ws, 0)
    assert e.value.status == sd.SD_EINVAL
    assert list(heads) == [5, 6, 7, 8, 9, 10, 11, 12] and l.n_full == 10


@pytest.mark.parametrize("case,status", [
    (dict(batch=1), sd.SD_EINVAL),
    (dict(batch=9), sd.SD_EINVAL),
    (dict(mode=sd.SD_KV_WINDOW), sd.SD_EINVAL),
    (dict(mode=sd.SD_PROJ_TEAL), sd.SD_EINVAL),
    (dict(ws_bytes=64), sd.SD_ENOSPC),
    (dict(full=True), sd.SD_ENOSPC),
    (dict(no_sel=True, mode=sd.SD_KV_SPARSE), sd.SD_EINVAL),
    (dict(dims=dict(d_model=8192)), sd.SD_EUNSUPPORTED),
    (dict(mode=sd.SD_MATRIX_CORES), sd.SD_EINVAL),           # no tile weights
    (dict(mode=sd.SD_MATRIX_CORES, dims=dict(w_dtype=sd.SD_F32)), sd.SD_EUNSUPPORTED),
    (dict(mode=1024), sd.SD_EINVAL),
])
def test_decode_step_batch_rejects_before_launch(case, status):
    batch = case.get("batch", 4)
    layers = (sd.sd_layer * 1)(sd.sd_layer(*([FAKE] * 7), 0.1, 0))
    kv = (sd.sd_seq_kv * batch)(*[sd.sd_seq_kv(FAKE, FAKE, 64, 10, None if case.get("no_sel") else FAKE,
                                              None if case.get("no_sel") else FAKE, 32, 5)
                                  for _ in range(batch)])
    if case.get("full"):
        kv[2].n_full = 64
    dims = _dims(**case.get("dims", {}))
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step_batch(dims, layers, kv, [10] * batch, FAKE, case.get("mode", 0),
                                _FakeWs(case.get("ws_bytes", 1 << 32)), 0)
    assert e.value.status == status
    assert all(k.n_full in (10, 64) and k.n_sel == 5 for k in kv)


def test_batch_workspace_grows_with_batch():
    a = sd.sd_batch_workspace_bytes(_dims(), 2)
    b = sd.sd_batch_workspace_bytes(_dims(), 8)
    assert 0 < a < b and sd.sd_batch_workspace_bytes(_dims(), 1) == 0


def test_noalloc_step_rejects_beyond_its_buffer_before_launch():
    # masked attention over 2^20 allocated rows needs 128 MiB of score rows,
    # more than the library's 64 MiB per-GPU buffer: refused on the host
    L = sd.sd_layer()
    L.cap_full = 1 << 20
    layers = (sd.sd_layer * 1)(L)
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step_noalloc(_dims(), layers, 0, FAKE, sd.SD_ATTN_MASKED, 0)
    assert e.value.status == sd.SD_ENOSPC
    assert sd.SD_NOALLOC_SCRATCH_BYTES == 64 << 20
    assert sd.sd_workspace_bytes(_dims(), 0, 0) <= sd.SD_NOALLOC_SCRATCH_BYTES


def test_batch_matrix_cores_accepts_tile_weights_alone():
    # with SD_MATRIX_CORES the row-major weights are not needed; a full cache
    # still stops the step on the host
    L = sd.sd_layer(attn_norm=FAKE, mlp_norm=FAKE, w_qkv_m=FAKE, w_o_m=FAKE, w_gate_m=FAKE,
                    w_up_m=FAKE, w_down_m=FAKE, cats_threshold=0.1)
    layers = (sd.sd_layer * 1)(L)
    kv = (sd.sd_seq_kv * 2)(sd.sd_seq_kv(FAKE, FAKE, 64, 10, None, None, 0, 0),
                            sd.sd_seq_kv(FAKE, FAKE, 64, 64, None, None, 0, 0))
    with pytest.raises(sd.SdError) as e:
        sd.sd_decode_step_batch(_dims(), layers, kv, [10, 64], FAKE, sd.SD_MATRIX_CORES,
                                _FakeWs(1 << 32), 0)
    assert e.value.status == sd.SD_ENOSPC and "sequence 1" in sd.sd_last_error()


@pytest.mark.parametrize("case", [
    dict(w=None), dict(out=None), dict(w=FAKE + 8), dict(rows=0), dict(d_in=12), dict(d_in=0),
    dict(out=FAKE + 4096),   # overlaps w
])
def test_pack_tiles_rejects_before_launch(case):
    args = dict(w=FAKE, rows=64, d_in=256, out=FAKE + (1 << 24))
    args.update(case)
    with pytest.raises(sd.SdError) as e:
        sd.sd_pack_tiles(args["w"], args["rows"], args["d_in"], args["out"], 0)
    assert e.value.status == sd.SD_EINVAL


def test_tile_bytes_pads_rows_and_channels():
    assert sd.sd_tile_bytes(16, 32) == 1024
    assert sd.sd_tile_bytes(17, 32) == 2048
    assert sd.sd_tile_bytes(16, 40) == 2048
    assert sd.sd_tile_bytes(6144, 4096) == 6144 * 4096 * 2


@pytest.mark.parametrize("case", [dict(buf=None), dict(buf=FAKE + 8), dict(nbytes=0),
                                  dict(nbytes=8192 + 16), dict(out=None)])
def test_stream_read_rejects_before_launch(case):
    args = dict(buf=FAKE, nbytes=1 << 20, out=FAKE + (1 << 24))
    args.update(case)
    with pytest.raises(sd.SdError) as e:
        sd.sd_stream_read(args["buf"], args["nbytes"], args["out"], 0)
    assert e.value.status == sd.SD_EINVAL
