"""Python binding of libmoeq: the routed-expert MoE forward over 4-bit codebook experts.

Argument marshalling only. Every step of the forward runs in the HIP kernels of libmoeq.so;
PyTorch provides device memory and the current stream. Importing fails loudly when the
library has not been built (``python -m codebook_quantized_moe_amd.build`` or
``__graft_entry__.build()``): there is no fallback.

The functions carry the C names of include/moeq.h and take torch tensors in place of device
pointers (``tables`` is a host numpy array or CPU tensor [n_tables, 8] fp32). A nonzero
status raises ``MoeqError`` with the library's message.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # noqa: F401  (loads the HIP runtime libmoeq links against before libmoeq itself)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmoeq.so is not built ({LIB_PATH}); run codebook_quantized_moe_amd/build.py")

_lib = ctypes.CDLL(LIB_PATH)

MOEQ_OK, MOEQ_EINVAL, MOEQ_EUNSUPPORTED, MOEQ_EWORKSPACE, MOEQ_ELAUNCH = 0, -1, -2, -3, -4
MOEQ_GATING_SOFTMAX_TOPK, MOEQ_GATING_SIGMOID_TOPK = 0, 1
MOEQ_STATIC_SCRATCH_BYTES = (32 << 20) + 256    # include/moeq.h
MAX_EXPERTS = 256
MAX_TABLES = 4

EXPORTED = ("moeq_last_error", "moeq_workspace_bytes", "moeq_router_logits", "moeq_route_topk",
            "moeq_permute_by_expert", "moeq_route_permute", "moeq_gateup_swiglu",
            "moeq_gateup_swiglu_static", "moeq_down",
            "moeq_unpermute_combine", "moeq_shared_workspace_bytes", "moeq_shared_expert",
            "moeq_unpermute_combine_shared", "moeq_quantize", "moeq_lloyd_workspace_bytes",
            "moeq_lloyd_stats", "moeq_lloyd_update", "moeq_select_arms",
            "moeq_moe_decode_workspace_bytes",
            "moeq_moe_decode", "moeq_moe_decode_check", "moeq_debug_dequant")

_i, _vp, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_lib.moeq_last_error.restype = ctypes.c_char_p
_lib.moeq_last_error.argtypes = []
_lib.moeq_workspace_bytes.restype = _sz
_lib.moeq_workspace_bytes.argtypes = [_i] * 5
_lib.moeq_router_logits.restype = _i
_lib.moeq_router_logits.argtypes = [_vp, _i, _i, _vp, _i, _vp, _vp]
_lib.moeq_route_topk.restype = _i
_lib.moeq_route_topk.argtypes = [_vp, _i, _i, _i, _i, _vp, _vp, _vp]
_lib.moeq_route_permute.restype = _i
_lib.moeq_route_permute.argtypes = [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.moeq_permute_by_expert.restype = _i
_lib.moeq_permute_by_expert.argtypes = [_vp, _i, _i, _i, _vp, _vp, _vp, _vp]
_lib.moeq_gateup_swiglu.restype = _i
_lib.moeq_gateup_swiglu.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _i, _vp, _vp, _vp, _sz, _vp]
_lib.moeq_gateup_swiglu_static.restype = _i
_lib.moeq_gateup_swiglu_static.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _i, _vp, _vp, _vp]
_lib.moeq_down.restype = _i
_lib.moeq_down.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp,
                           _vp, _sz, _vp]
_lib.moeq_unpermute_combine.restype = _i
_lib.moeq_unpermute_combine.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp]
_lib.moeq_shared_workspace_bytes.restype = _sz
_lib.moeq_shared_workspace_bytes.argtypes = [_i] * 3
_lib.moeq_shared_expert.restype = _i
_lib.moeq_shared_expert.argtypes = [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp,
                                    _vp, _vp, _vp, _sz, _vp]
_lib.moeq_unpermute_combine_shared.restype = _i
_lib.moeq_unpermute_combine_shared.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp]
_ll, _f = ctypes.c_longlong, ctypes.c_float
_lib.moeq_quantize.restype = _i
_lib.moeq_quantize.argtypes = [_vp, _i, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp]
_lib.moeq_lloyd_workspace_bytes.restype = _sz
_lib.moeq_lloyd_workspace_bytes.argtypes = [_i, _i]
_lib.moeq_lloyd_stats.restype = _i
_lib.moeq_lloyd_stats.argtypes = [_vp, _i, _i, _i, _vp, _f, _i, _vp, _vp, _sz, _vp]
_lib.moeq_lloyd_update.restype = _i
_lib.moeq_lloyd_update.argtypes = [_vp, _vp, _vp, _vp]
_lib.moeq_select_arms.restype = _i
_lib.moeq_select_arms.argtypes = [_vp, _vp, _i, _i, _i, _vp, _vp, _vp]
_lib.moeq_moe_decode_workspace_bytes.restype = _sz
_lib.moeq_moe_decode_workspace_bytes.argtypes = [_i] * 5
_lib.moeq_moe_decode.restype = _i
_lib.moeq_moe_decode.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _i, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moeq_moe_decode_check.restype = _i
_lib.moeq_moe_decode_check.argtypes = [_vp, _vp]
_lib.moeq_debug_dequant.restype = _i
_lib.moeq_debug_dequant.argtypes = [_vp, _vp, _i, _i, _i, _vp, _i, _vp, _vp, _vp]


class MoeqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libmoeq status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != MOEQ_OK:
        raise MoeqError(status, _lib.moeq_last_error().decode())


def _p(t):
    """Device (or host) address of a tensor / array, or None."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _tables(tables):
    a = np.ascontiguousarray(np.asarray(tables, dtype=np.float32).reshape(-1, 8))
    return a, a.shape[0]


def moeq_last_error() -> str:
    return _lib.moeq_last_error().decode()


def moeq_workspace_bytes(T: int, k: int, E: int, H: int, I: int) -> int:
    return int(_lib.moeq_workspace_bytes(T, k, E, H, I))


def moeq_router_logits(x, T, H, router_w, E, logits, stream=None):
    _check(_lib.moeq_router_logits(_p(x), T, H, _p(router_w), E, _p(logits), _stream(stream)))


def moeq_route_topk(logits, T, E, k, topk_ids, topk_w, gating=MOEQ_GATING_SOFTMAX_TOPK,
                    stream=None):
    _check(_lib.moeq_route_topk(_p(logits), T, E, k, gating, _p(topk_ids), _p(topk_w),
                                _stream(stream)))


def moeq_route_permute(logits, T, E, k, topk_ids, topk_w, expert_offsets, sorted_pair, pair_pos,
                       gating=MOEQ_GATING_SOFTMAX_TOPK, stream=None):
    _check(_lib.moeq_route_permute(_p(logits), T, E, k, gating, _p(topk_ids), _p(topk_w),
                                   _p(expert_offsets), _p(sorted_pair), _p(pair_pos),
                                   _stream(stream)))


def moeq_permute_by_expert(topk_ids, T, k, E, expert_offsets, sorted_pair, pair_pos,
                           stream=None):
    _check(_lib.moeq_permute_by_expert(_p(topk_ids), T, k, E, _p(expert_offsets),
                                       _p(sorted_pair), _p(pair_pos), _stream(stream)))


def moeq_gateup_swiglu(x, T, H, I, E, k, expert_offsets, sorted_pair, gate_codes, gate_scales,
                       up_codes, up_scales, tables, table_id, inter, ws=None, ws_bytes=0,
                       stream=None):
    tab, n = _tables(tables)
    _check(_lib.moeq_gateup_swiglu(_p(x), T, H, I, E, k, _p(expert_offsets), _p(sorted_pair),
                                   _p(gate_codes), _p(gate_scales), _p(up_codes), _p(up_scales),
                                   tab.ctypes.data, n, _p(table_id), _p(inter), _p(ws), ws_bytes,
                                   _stream(stream)))


def moeq_gateup_swiglu_static(x, T, H, I, E, k, expert_offsets, sorted_pair, gate_codes,
                              gate_scales, up_codes, up_scales, tables, table_id, inter,
                              stream=None):
    tab, n = _tables(tables)
    _check(_lib.moeq_gateup_swiglu_static(_p(x), T, H, I, E, k, _p(expert_offsets),
                                          _p(sorted_pair), _p(gate_codes), _p(gate_scales),
                                          _p(up_codes), _p(up_scales), tab.ctypes.data, n,
                                          _p(table_id), _p(inter), _stream(stream)))


def moeq_down(inter, T, H, I, E, k, expert_offsets, sorted_pair, topk_w, down_codes,
              down_scales, tables, table_id, yp, ws=None, ws_bytes=0, stream=None):
    tab, n = _tables(tables)
    _check(_lib.moeq_down(_p(inter), T, H, I, E, k, _p(expert_offsets), _p(sorted_pair),
                          _p(topk_w), _p(down_codes), _p(down_scales), tab.ctypes.data, n,
                          _p(table_id), _p(yp), _p(ws), ws_bytes, _stream(stream)))


def moeq_unpermute_combine(yp, pair_pos, expert_offsets, T, k, E, H, residual, y, stream=None):
    _check(_lib.moeq_unpermute_combine(_p(yp), _p(pair_pos), _p(expert_offsets), T, k, E, H,
                                       _p(residual), _p(y), _stream(stream)))


def moeq_shared_workspace_bytes(T: int, H: int, I: int) -> int:
    return int(_lib.moeq_shared_workspace_bytes(T, H, I))


def moeq_shared_expert(x, T, H, I, gate_codes, gate_scales, up_codes, up_scales, down_codes,
                       down_scales, tables, table_id, inter, z, ws, ws_bytes, stream=None):
    tab, n = _tables(tables)
    _check(_lib.moeq_shared_expert(_p(x), T, H, I, _p(gate_codes), _p(gate_scales), _p(up_codes),
                                   _p(up_scales), _p(down_codes), _p(down_scales), tab.ctypes.data,
                                   n, _p(table_id), _p(inter), _p(z), _p(ws), ws_bytes,
                                   _stream(stream)))


def moeq_unpermute_combine_shared(yp, pair_pos, expert_offsets, T, k, E, H, shared_z, residual,
                                  y, stream=None):
    _check(_lib.moeq_unpermute_combine_shared(_p(yp), _p(pair_pos), _p(expert_offsets), T, k, E,
                                              H, _p(shared_z), _p(residual), _p(y),
                                              _stream(stream)))


def moeq_quantize(w, E, N, K, tables, table_id, codes, scales, row_err, stream=None):
    tab, n = _tables(tables)
    _check(_lib.moeq_quantize(_p(w), E, N, K, tab.ctypes.data, n, _p(table_id), _p(codes),
                              _p(scales), _p(row_err), _stream(stream)))


def moeq_lloyd_workspace_bytes(E: int, N: int) -> int:
    return int(_lib.moeq_lloyd_workspace_bytes(E, N))


def moeq_lloyd_stats(w, E, N, K, table, gmax, accumulate, stats, ws, ws_bytes, stream=None):
    tab = np.ascontiguousarray(np.asarray(table, dtype=np.float32).reshape(8))
    _check(_lib.moeq_lloyd_stats(_p(w), E, N, K, tab.ctypes.data, float(gmax),
                                 1 if accumulate else 0, _p(stats), _p(ws), ws_bytes,
                                 _stream(stream)))


def moeq_lloyd_update(stats, table):
    """stats: host float64 [24] from moeq_lloyd_stats; table: the 8 magnitudes they were taken
    against. Returns (next fp32 table [8], weighted squared error of the assignment)."""
    st = np.ascontiguousarray(np.asarray(stats, dtype=np.float64).reshape(24))
    tab = np.ascontiguousarray(np.asarray(table, dtype=np.float32).reshape(8))
    nxt = np.empty(8, np.float32)
    err = ctypes.c_double(0.0)
    _check(_lib.moeq_lloyd_update(st.ctypes.data, tab.ctypes.data, nxt.ctypes.data,
                                  ctypes.addressof(err)))
    return nxt, err.value


def moeq_select_arms(err_a, err_b, E, N, accumulate, table_id, expert_err, stream=None):
    _check(_lib.moeq_select_arms(_p(err_a), _p(err_b), E, N, 1 if accumulate else 0,
                                 _p(table_id), _p(expert_err), _stream(stream)))


def moeq_moe_decode_workspace_bytes(T: int, k: int, E: int, H: int, I: int) -> int:
    return int(_lib.moeq_moe_decode_workspace_bytes(T, k, E, H, I))


def moeq_moe_decode(x, logits, T, H, I, E, k, gate_codes, gate_scales, up_codes, up_scales,
                    down_codes, down_scales, tables, table_id, residual, y, ws, ws_bytes,
                    gating=MOEQ_GATING_SOFTMAX_TOPK, stream=None):
    tab, n = _tables(tables)
    _check(_lib.moeq_moe_decode(_p(x), _p(logits), T, H, I, E, k, gating, _p(gate_codes),
                                _p(gate_scales), _p(up_codes), _p(up_scales), _p(down_codes),
                                _p(down_scales), tab.ctypes.data, n, _p(table_id), _p(residual),
                                _p(y), _p(ws), ws_bytes, _stream(stream)))


def moeq_moe_decode_check(ws, stream=None):
    _check(_lib.moeq_moe_decode_check(_p(ws), _stream(stream)))


def moeq_debug_dequant(codes, scales, E, N, K, tables, table_id, out, stream=None):
    tab, n = _tables(tables)
    _check(_lib.moeq_debug_dequant(_p(codes), _p(scales), E, N, K, tab.ctypes.data, n,
                                   _p(table_id), _p(out), _stream(stream)))


def inter_slot(c):
    """Position of intermediate channel c in a row of ``inter`` (moeq_inter_slot)."""
    c = np.asarray(c)
    return (c & ~7) | (((c & 1) << 2) | ((c & 7) >> 1))


from .layer import MoeLayer, DeviceWeights  # noqa: E402,F401
