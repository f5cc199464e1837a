"""Python binding of libsd.so, the MI355X sparse decode-step library.

Argument marshalling only: every function here forwards to the C entry point
of the same name in include/sd.h, passing device pointers of torch tensors
(torch provides device memory and streams) and raising SdError on a non-OK
status.  There is no fallback: if libsd.so is missing the import fails.
"""

from __future__ import annotations

import ctypes
import os

# torch brings its own HIP runtime (same soname as ROCm's).  Load it first so
# that libsd.so binds to the runtime that owns the tensors' device memory.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsd.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")

_lib = ctypes.CDLL(LIB_PATH)

SD_OK, SD_EINVAL, SD_ENOSPC, SD_EUNSUPPORTED, SD_EHIP = range(5)
SD_F32, SD_BF16 = 0, 1
SD_SCORES_IN, SD_GATE_IN, SD_KV_SPARSE, SD_MLP_SPARSE = 1, 2, 4, 8
SD_KV_WINDOW, SD_ATTN_MASKED, SD_ATTN_FUSED = 16, 32, 64
SD_PROJ_TEAL, SD_ACCUMULATE, SD_MATRIX_CORES = 128, 256, 512
SD_PROJ_ALL7, SD_PROJ_FFN, SD_PROJ_CATS = 0, 1, 2

EXPORTS = ("sd_workspace_bytes", "sd_select_kv", "sd_select_kv_ragged", "sd_decode_attn",
           "sd_decode_attn_ragged", "sd_decode_attn_window",
           "sd_decode_attn_baseline", "sd_sparse_mlp", "sd_teal_gemv",
           "sd_decode_step", "sd_decode_step_noalloc", "sd_batch_workspace_bytes", "sd_decode_step_batch", "sd_byte_account",
           "sd_pack_tiles", "sd_stream_read", "sd_byte_crossover_batch", "sd_latency_fit", "sd_latency_crossing", "sd_latency_gate",
           "sd_calibrate_workspace_bytes",
           "sd_cats_calibrate", "sd_profile_start", "sd_profile_stop", "sd_status_string",
           "sd_last_error")


class sd_dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float)]


class sd_layer(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p), ("mlp_norm", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down_t", ctypes.c_void_p), ("cats_threshold", ctypes.c_float),
                ("pad0", ctypes.c_int32),
                ("k_full", ctypes.c_void_p), ("v_full", ctypes.c_void_p),
                ("cap_full", ctypes.c_int32), ("n_full", ctypes.c_int32),
                ("k_sel", ctypes.c_void_p), ("v_sel", ctypes.c_void_p),
                ("cap_sel", ctypes.c_int32), ("n_sel", ctypes.c_int32),
                ("mask_out", ctypes.c_void_p), ("window_keep", ctypes.c_int32),
                ("window_sink", ctypes.c_int32),
                ("w_qkv_t", ctypes.c_void_p), ("w_o_t", ctypes.c_void_p),
                ("w_gate_t", ctypes.c_void_p), ("w_up_t", ctypes.c_void_p),
                ("teal_t", ctypes.c_float * 4), ("teal_masks_out", ctypes.c_void_p),
                ("n_sel_heads", ctypes.POINTER(ctypes.c_int32)),
                ("w_qkv_m", ctypes.c_void_p), ("w_o_m", ctypes.c_void_p),
                ("w_gate_m", ctypes.c_void_p), ("w_up_m", ctypes.c_void_p),
                ("w_down_m", ctypes.c_void_p), ("w_down_b", ctypes.c_void_p)]


class sd_seq_kv(ctypes.Structure):
    _fields_ = [("k_full", ctypes.c_void_p), ("v_full", ctypes.c_void_p),
                ("cap_full", ctypes.c_int32), ("n_full", ctypes.c_int32),
                ("k_sel", ctypes.c_void_p), ("v_sel", ctypes.c_void_p),
                ("cap_sel", ctypes.c_int32), ("n_sel", ctypes.c_int32)]


class sd_byte_record(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in
                ("b_attn", "b_mlp", "b_kv", "b_total", "delta_p", "delta_kv", "bound_p",
                 "bound_kv", "bound_both", "n_star", "n_star_budget", "gap_per_k", "n_lat")]


class sd_latency_model(ctypes.Structure):
    _fields_ = [("bw_eff", ctypes.c_double), ("c_p", ctypes.c_double), ("c_kv", ctypes.c_double)]


class sd_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32),
                ("pad0", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_U = ctypes.c_uint32
_F = ctypes.c_float
_D = ctypes.c_double
_S = ctypes.c_size_t

_lib.sd_workspace_bytes.restype = _S
_lib.sd_workspace_bytes.argtypes = [ctypes.POINTER(sd_dims), _I, _I]
_lib.sd_select_kv.restype = _I
_lib.sd_select_kv.argtypes = [ctypes.POINTER(sd_dims), _P, _P, _I, _I, _P, _I, _I, _I, _P, _P,
                              _P, _P, _I, _U, _P, _S, _P]
_lib.sd_select_kv_ragged.restype = _I
_lib.sd_select_kv_ragged.argtypes = [ctypes.POINTER(sd_dims), _P, _P, _I, _I, _P, _I, _I,
                                     ctypes.POINTER(_I), _P, _P, _I, _P, _P, _I, _U, _P, _S, _P]
_lib.sd_decode_attn_ragged.restype = _I
_lib.sd_decode_attn_ragged.argtypes = [ctypes.POINTER(sd_dims), _P, _P, _P, _I,
                                       ctypes.POINTER(_I), _F, _I, _P, _P, _P, _S, _P]
_lib.sd_batch_workspace_bytes.restype = _S
_lib.sd_batch_workspace_bytes.argtypes = [ctypes.POINTER(sd_dims), _I]
_lib.sd_decode_step_batch.restype = _I
_lib.sd_decode_step_batch.argtypes = [ctypes.POINTER(sd_dims), _I, ctypes.POINTER(sd_layer), _I,
                                      ctypes.POINTER(sd_seq_kv), ctypes.POINTER(_I), _P, _U, _P,
                                      _S, _P]
_lib.sd_stream_read.restype = _I
_lib.sd_stream_read.argtypes = [_P, _S, _P, _P]
SD_STREAM_BLOCKS = 2048
_lib.sd_pack_tiles.restype = _I
_lib.sd_pack_tiles.argtypes = [_P, _I, _I, _P, _P]
_lib.sd_decode_attn.restype = _I
_lib.sd_decode_attn.argtypes = [ctypes.POINTER(sd_dims), _P, _P, _P, _I, _I, _F, _I, _P, _P,
                                _P, _S, _P]
_lib.sd_decode_attn_window.restype = _I
_lib.sd_decode_attn_window.argtypes = [ctypes.POINTER(sd_dims), _P, _P, _P, _I, _I, _I, _I, _F,
                                       _I, _P, _P, _P, _S, _P]
_lib.sd_decode_attn_baseline.restype = _I
_lib.sd_decode_attn_baseline.argtypes = [ctypes.POINTER(sd_dims), _P, _P, _P, _I, _I, _F, _I, _P,
                                         _P, _P, _S, _P]
_lib.sd_sparse_mlp.restype = _I
_lib.sd_sparse_mlp.argtypes = [ctypes.POINTER(sd_dims), _P, _P, _P, _P, _P, _F, _P, _P, _P, _P,
                               _U, _P, _S, _P]
_lib.sd_teal_gemv.restype = _I
_lib.sd_teal_gemv.argtypes = [ctypes.POINTER(sd_dims), _P, _I, _P, _F, _P, _P, _I, _P, _P, _U,
                              _P, _P, _P, _S, _P]
_lib.sd_decode_step.restype = _I
_lib.sd_decode_step.argtypes = [ctypes.POINTER(sd_dims), _I, ctypes.POINTER(sd_layer), _I, _P,
                                _U, _P, _S, _P]
_lib.sd_decode_step_noalloc.restype = _I
_lib.sd_decode_step_noalloc.argtypes = [ctypes.POINTER(sd_dims), _I, ctypes.POINTER(sd_layer), _I,
                                        _P, _U, _P]
SD_NOALLOC_SCRATCH_BYTES = 64 << 20
_lib.sd_byte_account.restype = _I
_lib.sd_byte_account.argtypes = [ctypes.POINTER(sd_dims), _I, _D, _D, _D, _D, _D, _I, _D,
                                 ctypes.POINTER(sd_latency_model), ctypes.POINTER(sd_byte_record)]
_DP = ctypes.POINTER(_D)
_lib.sd_latency_fit.restype = _I
_lib.sd_latency_fit.argtypes = [_I, _DP, _DP, _I, _DP, _DP, _DP, _DP]
_lib.sd_latency_crossing.restype = _I
_lib.sd_latency_crossing.argtypes = [_I, _DP, _DP, _DP, _DP]
_lib.sd_latency_gate.restype = _I
_lib.sd_latency_gate.argtypes = [_I, _DP, _DP, ctypes.POINTER(ctypes.c_uint8), _D,
                                 ctypes.POINTER(_I)]
_lib.sd_calibrate_workspace_bytes.restype = _S
_lib.sd_calibrate_workspace_bytes.argtypes = [ctypes.POINTER(sd_dims), _I]
_lib.sd_cats_calibrate.restype = _I
_lib.sd_cats_calibrate.argtypes = [ctypes.POINTER(sd_dims), _P, _I, _P, _P, _F, _P, _P, _S, _P]
_lib.sd_profile_start.restype = _I
_lib.sd_profile_start.argtypes = []
_lib.sd_profile_stop.restype = _I
_lib.sd_profile_stop.argtypes = [ctypes.POINTER(sd_kernel_stat), _I]
_lib.sd_status_string.restype = ctypes.c_char_p
_lib.sd_status_string.argtypes = [_I]
_lib.sd_last_error.restype = ctypes.c_char_p
_lib.sd_last_error.argtypes = []


class SdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_lib.sd_status_string(status).decode()}: {message}")
        self.status = status


def _check(status: int) -> None:
    if status != SD_OK:
        raise SdError(status, _lib.sd_last_error().decode())


def _ptr(x):
    """Device pointer of a tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws):
    """(pointer, bytes) of a workspace tensor."""
    return _ptr(ws), ws.numel() * ws.element_size()


def make_dims(d_model, n_q_heads, n_kv_heads, head_dim, d_ff, w_dtype, kv_dtype,
              rms_eps=1e-5, rope_theta=500000.0) -> sd_dims:
    return sd_dims(d_model, n_q_heads, n_kv_heads, head_dim, d_ff, w_dtype, kv_dtype,
                   rms_eps, rope_theta)


def sd_workspace_bytes(dims: sd_dims, max_rows: int, max_window: int) -> int:
    return int(_lib.sd_workspace_bytes(ctypes.byref(dims), max_rows, max_window))


def sd_select_kv(dims, k_full, v_full, cap_full, n, q_window, w, n_sink, k_keep, scores, idx,
                 k_sel, v_sel, cap_sel, flags, ws, stream=None) -> None:
    p, nb = _ws(ws)
    _check(_lib.sd_select_kv(ctypes.byref(dims), _ptr(k_full), _ptr(v_full), cap_full, n,
                             _ptr(q_window), w, n_sink, k_keep, _ptr(scores), _ptr(idx),
                             _ptr(k_sel), _ptr(v_sel), cap_sel, flags, p, nb, _stream(stream)))


def _host_ints(vals):
    vals = [int(x) for x in vals]
    return (_I * max(1, len(vals)))(*vals)


def sd_select_kv_ragged(dims, k_full, v_full, cap_full, n, q_window, w, n_sink, k_keep_heads,
                        scores, idx, idx_stride, k_sel, v_sel, cap_sel, flags, ws,
                        stream=None) -> None:
    p, nb = _ws(ws)
    _check(_lib.sd_select_kv_ragged(ctypes.byref(dims), _ptr(k_full), _ptr(v_full), cap_full, n,
                                    _ptr(q_window), w, n_sink, _host_ints(k_keep_heads),
                                    _ptr(scores), _ptr(idx), idx_stride, _ptr(k_sel), _ptr(v_sel),
                                    cap_sel, flags, p, nb, _stream(stream)))


def sd_decode_attn_ragged(dims, q, k, v, cap, n_ctx_heads, scale, n_splits, out, lse, ws,
                          stream=None) -> None:
    p, nb = _ws(ws)
    _check(_lib.sd_decode_attn_ragged(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), cap,
                                      _host_ints(n_ctx_heads), scale, n_splits, _ptr(out),
                                      _ptr(lse), p, nb, _stream(stream)))


def sd_decode_attn(dims, q, k, v, cap, n_ctx, scale, n_splits, out, lse, ws, stream=None) -> None:
    p, nb = _ws(ws)
    _check(_lib.sd_decode_attn(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), cap, n_ctx, scale,
                               n_splits, _ptr(out), _ptr(lse), p, nb, _stream(stream)))


def sd_decode_attn_window(dims, q, k, v, cap, n_rows, n_sink, n_keep, scale, n_splits, out, lse,
                          ws, stream=None) -> None:
    p, nb = _ws(ws)
    _check(_lib.sd_decode_attn_window(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), cap, n_rows,
                                      n_sink, n_keep, scale, n_splits, _ptr(out), _ptr(lse), p,
                                      nb, _stream(stream)))


def sd_decode_attn_baseline(dims, q, k, v, cap, n_ctx, scale, path, out, lse, ws,
                            stream=None) -> None:
    p, nb = _ws(ws)
    _check(_lib.sd_decode_attn_baseline(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), cap, n_ctx,
                                        scale, path, _ptr(out), _ptr(lse), p, nb,
                                        _stream(stream)))


def sd_sparse_mlp(dims, x, norm_w, w_gate, w_up, w_down_t, threshold, y, act, idx, n_kept,
                  flags, ws, stream=None) -> None:
    p, nb = _ws(ws)
    _check(_lib.sd_sparse_mlp(ctypes.byref(dims), _ptr(x), _ptr(norm_w), _ptr(w_gate), _ptr(w_up),
                              _ptr(w_down_t), threshold, _ptr(y), _ptr(act), _ptr(idx),
                              _ptr(n_kept), flags, p, nb, _stream(stream)))


def sd_teal_gemv(dims, x, d_in, norm_w, threshold, w_t, w2_t, d_out, y, y2, flags, idx, n_kept,
                 ws, stream=None) -> None:
    p, nb = _ws(ws)
    _check(_lib.sd_teal_gemv(ctypes.byref(dims), _ptr(x), d_in, _ptr(norm_w), threshold, _ptr(w_t),
                             _ptr(w2_t), d_out, _ptr(y), _ptr(y2), flags, _ptr(idx), _ptr(n_kept),
                             p, nb, _stream(stream)))


def sd_batch_workspace_bytes(dims: sd_dims, batch: int) -> int:
    return int(_lib.sd_batch_workspace_bytes(ctypes.byref(dims), batch))


def sd_decode_step_batch(dims, layers, kv, pos, hidden, mode, ws, stream=None) -> None:
    """`layers`: ctypes array of sd_layer [n_layers] (weights); `kv`: ctypes
    array of sd_seq_kv [batch * n_layers], sequence-major (advanced in place);
    `pos`: the batch's positions."""
    p, nb = _ws(ws)
    n_layers = len(layers)
    batch = len(kv) // n_layers if n_layers else 0
    _check(_lib.sd_decode_step_batch(ctypes.byref(dims), n_layers, layers, batch, kv,
                                     _host_ints(pos), _ptr(hidden), mode, p, nb,
                                     _stream(stream)))


def sd_tile_bytes(rows: int, d_in: int) -> int:
    """Bytes of a [rows, d_in] weight in the tile layout (SD_TILE_BYTES)."""
    return ((rows + 15) // 16) * ((d_in + 31) // 32) * 1024


def sd_stream_read(buf, nbytes, out, stream=None) -> None:
    """One plain read of nbytes of buf; out [SD_STREAM_BLOCKS] uint32/int32 checksums."""
    _check(_lib.sd_stream_read(_ptr(buf), nbytes, _ptr(out), _stream(stream)))


def sd_pack_tiles(w, rows, d_in, out, stream=None) -> None:
    _check(_lib.sd_pack_tiles(_ptr(w), rows, d_in, _ptr(out), _stream(stream)))


def sd_decode_step(dims, layers, pos, hidden, mode, ws, stream=None) -> None:
    """`layers` is a ctypes array of sd_layer (n_full/n_sel advance in place)."""
    p, nb = _ws(ws)
    _check(_lib.sd_decode_step(ctypes.byref(dims), len(layers), layers, pos, _ptr(hidden), mode,
                               p, nb, _stream(stream)))


def sd_decode_step_noalloc(dims, layers, pos, hidden, mode, stream=None) -> None:
    """sd_decode_step on the library's own per-GPU scratch buffer (no workspace)."""
    _check(_lib.sd_decode_step_noalloc(ctypes.byref(dims), len(layers), layers, pos,
                                       _ptr(hidden), mode, _stream(stream)))


def sd_byte_account(dims, n_layers, n, r_p, r_kv, s_w, s_kv, proj_set, fixed_bytes=0.0,
                    latency=None):
    """`latency`: None or (bw_eff bytes/s, c_p s, c_kv s) for gap_per_k and n_lat."""
    rec = sd_byte_record()
    lat = None if latency is None else ctypes.byref(sd_latency_model(*latency))
    _check(_lib.sd_byte_account(ctypes.byref(dims), n_layers, n, r_p, r_kv, s_w, s_kv, proj_set,
                                fixed_bytes, lat, ctypes.byref(rec)))
    return rec


def _host_doubles(vals):
    vals = [float(x) for x in vals]
    return (_D * max(1, len(vals)))(*vals)


def sd_latency_fit(bytes_dense, t_dense, bytes_modes, t_modes):
    """(bw_eff, [c per mode]) from a sweep: `bytes_modes`/`t_modes` are one
    list per mode, each as long as `bytes_dense`."""
    npts, nm = len(bytes_dense), len(bytes_modes)
    bw = _D()
    c = (_D * max(1, nm))()
    _check(_lib.sd_latency_fit(npts, _host_doubles(bytes_dense), _host_doubles(t_dense), nm,
                               _host_doubles([x for row in bytes_modes for x in row]),
                               _host_doubles([x for row in t_modes for x in row]),
                               ctypes.byref(bw), c))
    return bw.value, [c[i] for i in range(nm)]


def sd_latency_crossing(ctx, t_a, t_b) -> float:
    out = _D()
    _check(_lib.sd_latency_crossing(len(ctx), _host_doubles(ctx), _host_doubles(t_a),
                                    _host_doubles(t_b), ctypes.byref(out)))
    return out.value


def sd_latency_gate(t_step, t_once, horizon, admissible=None) -> int:
    best = _I()
    adm = None
    if admissible is not None:
        adm = (ctypes.c_uint8 * max(1, len(admissible)))(*[1 if a else 0 for a in admissible])
    _check(_lib.sd_latency_gate(len(t_step), _host_doubles(t_step), _host_doubles(t_once), adm,
                                horizon, ctypes.byref(best)))
    return best.value


_lib.sd_byte_crossover_batch.restype = _I
_lib.sd_byte_crossover_batch.argtypes = [ctypes.POINTER(sd_dims), _I, _D, _D, _D, _D, _I,
                                         ctypes.POINTER(_D)]


def sd_byte_crossover_batch(dims, batch, u_b, r_kv, s_w, s_kv, proj_set) -> float:
    out = _D()
    _check(_lib.sd_byte_crossover_batch(ctypes.byref(dims), batch, u_b, r_kv, s_w, s_kv, proj_set,
                                        ctypes.byref(out)))
    return out.value


def sd_calibrate_workspace_bytes(dims, n_states) -> int:
    return int(_lib.sd_calibrate_workspace_bytes(ctypes.byref(dims), n_states))


def sd_cats_calibrate(dims, states, n_states, norm_w, w_gate, sparsity, threshold, ws,
                      stream=None) -> None:
    p, nb = _ws(ws)
    _check(_lib.sd_cats_calibrate(ctypes.byref(dims), _ptr(states), n_states, _ptr(norm_w),
                                  _ptr(w_gate), sparsity, _ptr(threshold), p, nb,
                                  _stream(stream)))


def sd_profile_start() -> None:
    _check(_lib.sd_profile_start())


def sd_profile_stop() -> dict:
    """{kernel kind: (launches, total ms)} recorded since sd_profile_start()."""
    buf = (sd_kernel_stat * 32)()
    n = _lib.sd_profile_stop(buf, 32)
    if n < 0:
        raise SdError(SD_EHIP, "profiling event query failed")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n, 32))}


def sd_status_string(status: int) -> str:
    return _lib.sd_status_string(status).decode()


def sd_last_error() -> str:
    return _lib.sd_last_error().decode()
