"""ctypes binding of libmoe.so: the five layer calls plus helpers, same names as the C ABI.

Argument marshalling only.  Tensor arguments are torch tensors on the GPU (or
raw integer device addresses, or None for NULL); the stream defaults to torch's
current stream.  Every call raises MoeError on a non-zero status.  There is no
fallback: if libmoe.so is missing the import of the library raises.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = 0, -1, -2, -3, -4, -5
MOE_ERR_SCRATCH = -6
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_SCORES_IN = 1
MOE_FFN_ALL, MOE_FFN_GATE_UP, MOE_FFN_DOWN = 0, 1, 2
MOE_WS_DISPATCH, MOE_WS_FFN, MOE_WS_FFN_BWD, MOE_WS_ROUTE_BWD, MOE_WS_ROUTE = 1, 2, 3, 4, 5
MOE_WSP_H, MOE_WSP_H_SCALE, MOE_WSP_H_SHARED, MOE_WSP_H_SHARED_SCALE = 0, 1, 2, 3
_DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8_e4m3": MOE_FP8_E4M3}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


class MoeCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "E", "G", "M", "k", "S", "I", "group_topr")] + [
        ("route_scale", ctypes.c_float), ("act", ctypes.c_int32), ("wgt", ctypes.c_int32),
        ("bias_eq_mode", ctypes.c_int32)]


class MoeExpertWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_gate_up", "w_down", "w_gate_up_scale", "w_down_scale",
        "ws_gate_up", "ws_down", "ws_gate_up_scale", "ws_down_scale")]


class MoeExpertGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gate_up", "w_down", "ws_gate_up", "ws_down")]


class MoeFfnSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("g", "u", "gs", "us")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built by biased_top_routing_amd.build); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run python -m biased_top_routing_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
        cfgp = ctypes.POINTER(MoeCfg)
        sig = {
            "moe_route": [cfgp, vp, vp, vp, vp, vp, u32, vp, vp, vp, sz, vp],
            "moe_dispatch": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_dispatch_noalloc": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "moe_expert_ffn": [cfgp, vp, vp, vp, ctypes.POINTER(MoeExpertWeights), vp, vp, vp, vp, sz,
                               ctypes.c_int, vp],
            "moe_expert_ffn_gather": [cfgp, vp, vp, vp, ctypes.POINTER(MoeExpertWeights), vp, vp, vp, sz,
                                      ctypes.c_int, vp],
            "moe_expert_ffn_save": [cfgp, vp, vp, vp, ctypes.POINTER(MoeExpertWeights), vp, vp, vp,
                                    ctypes.POINTER(MoeFfnSaved), vp, sz, ctypes.c_int, vp],
            "moe_combine": [cfgp, vp, vp, vp, vp, vp, vp],
            "moe_combine_backward": [cfgp, vp, vp, vp, vp, vp, vp, vp],
            "moe_expert_ffn_backward": [cfgp, vp, vp, vp, ctypes.POINTER(MoeExpertWeights), vp, vp, vp, vp,
                                        ctypes.POINTER(MoeExpertGrads), vp, sz, vp],
            "moe_expert_ffn_backward_saved": [cfgp, vp, vp, vp, ctypes.POINTER(MoeExpertWeights),
                                              ctypes.POINTER(MoeFfnSaved), vp, vp, vp, vp,
                                              ctypes.POINTER(MoeExpertGrads), vp, sz, vp],
            "moe_route_backward": [cfgp, vp, vp, vp, vp, vp, f32, i32, vp, vp, vp, vp, sz, vp],
            "moe_dispatch_backward": [cfgp, vp, vp, vp, vp, vp, vp],
            "moe_update_bias": [cfgp, vp, vp, f32, vp],
            "moe_quantize_fp8": [vp, i32, i32, i32, i32, vp, vp, vp],
            "moe_ffn_workspace_part": [cfgp, ctypes.c_int, ctypes.POINTER(sz), ctypes.POINTER(sz)],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_workspace_bytes.argtypes = [cfgp, ctypes.c_int]
        L.moe_workspace_bytes.restype = sz
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/moe.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|size_t|const char\*|int)\s+(moe_\w+)\s*\(", text, re.M)))


def make_cfg(T, H, E, G, M, k, S, I, group_topr=2, route_scale=1.0, act="bf16", wgt="bf16",
             bias_eq_mode=0) -> MoeCfg:
    a = _DTYPES[act] if isinstance(act, str) else act
    w = _DTYPES[wgt] if isinstance(wgt, str) else wgt
    return MoeCfg(T, H, E, G, M, k, S, I, group_topr, route_scale, a, w, bias_eq_mode)


def cfg_from(c, **over) -> MoeCfg:
    """MoeCfg from any object with the layer attributes (T H E G M k S I group_topr
    route_scale act wgt bias_eq_mode)."""
    d = {n: getattr(c, n) for n in ("T", "H", "E", "G", "M", "k", "S", "I", "group_topr", "route_scale",
                                     "act", "wgt")}
    d["bias_eq_mode"] = getattr(c, "bias_eq_mode", 0)
    d.update(over)
    return make_cfg(**d)


def _p(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(name: str, st: int) -> None:
    if st != MOE_OK:
        raise MoeError(name, st)


def moe_route(cfg, x, w_router, logit_offset, bias, scores, flags, topk_idx, topk_w, ws=None, stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(cfg), _p(x), _p(w_router), _p(logit_offset), _p(bias),
                                        _p(scores), flags, _p(topk_idx), _p(topk_w), _p(ws), _nbytes(ws),
                                        _s(stream)))


def moe_dispatch(cfg, topk_idx, x, counts, offsets, perm, inv, x_perm, x_perm_scale, ws, stream=None):
    _check("moe_dispatch", lib().moe_dispatch(ctypes.byref(cfg), _p(topk_idx), _p(x), _p(counts), _p(offsets),
                                              _p(perm), _p(inv), _p(x_perm), _p(x_perm_scale), _p(ws),
                                              _nbytes(ws), _s(stream)))


def moe_dispatch_noalloc(cfg, topk_idx, x, counts, offsets, perm, inv, x_perm, x_perm_scale, stream=None):
    _check("moe_dispatch_noalloc", lib().moe_dispatch_noalloc(
        ctypes.byref(cfg), _p(topk_idx), _p(x), _p(counts), _p(offsets), _p(perm), _p(inv), _p(x_perm),
        _p(x_perm_scale), _s(stream)))


def expert_weights(w_gate_up, w_down, ws_gate_up=None, ws_down=None, w_gate_up_scale=None,
                   w_down_scale=None, ws_gate_up_scale=None, ws_down_scale=None) -> MoeExpertWeights:
    return MoeExpertWeights(_p(w_gate_up), _p(w_down), _p(w_gate_up_scale), _p(w_down_scale),
                            _p(ws_gate_up), _p(ws_down), _p(ws_gate_up_scale), _p(ws_down_scale))


def moe_expert_ffn(cfg, x_perm, x_perm_scale, offsets, weights: MoeExpertWeights, x, y_perm, y_shared, ws,
                   phase=MOE_FFN_ALL, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(ctypes.byref(cfg), _p(x_perm), _p(x_perm_scale), _p(offsets),
                                                  ctypes.byref(weights), _p(x), _p(y_perm), _p(y_shared),
                                                  _p(ws), _nbytes(ws), phase, _s(stream)))


def moe_expert_ffn_gather(cfg, x, perm, offsets, weights: MoeExpertWeights, y_perm, y_shared, ws,
                          phase=MOE_FFN_ALL, stream=None):
    _check("moe_expert_ffn_gather", lib().moe_expert_ffn_gather(
        ctypes.byref(cfg), _p(x), _p(perm), _p(offsets), ctypes.byref(weights), _p(y_perm), _p(y_shared),
        _p(ws), _nbytes(ws), phase, _s(stream)))


def ffn_saved(g, u, gs=None, us=None) -> MoeFfnSaved:
    return MoeFfnSaved(_p(g), _p(u), _p(gs), _p(us))


def moe_expert_ffn_save(cfg, x_perm, perm, offsets, weights: MoeExpertWeights, x, y_perm, y_shared,
                        saved: MoeFfnSaved, ws, phase=MOE_FFN_ALL, stream=None):
    _check("moe_expert_ffn_save", lib().moe_expert_ffn_save(
        ctypes.byref(cfg), _p(x_perm), _p(perm), _p(offsets), ctypes.byref(weights), _p(x), _p(y_perm),
        _p(y_shared), ctypes.byref(saved), _p(ws), _nbytes(ws), phase, _s(stream)))


def moe_combine(cfg, y_perm, y_shared, inv, topk_w, y, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(cfg), _p(y_perm), _p(y_shared), _p(inv), _p(topk_w),
                                            _p(y), _s(stream)))


def expert_grads(w_gate_up, w_down, ws_gate_up=None, ws_down=None) -> MoeExpertGrads:
    return MoeExpertGrads(_p(w_gate_up), _p(w_down), _p(ws_gate_up), _p(ws_down))


def moe_combine_backward(cfg, dy, y_perm, inv, topk_w, dy_perm, d_topk_w, stream=None):
    _check("moe_combine_backward", lib().moe_combine_backward(
        ctypes.byref(cfg), _p(dy), _p(y_perm), _p(inv), _p(topk_w), _p(dy_perm), _p(d_topk_w), _s(stream)))


def moe_expert_ffn_backward(cfg, x_perm, x, offsets, weights: MoeExpertWeights, dy_perm, dy, dx_perm, dx_shared,
                            grads: MoeExpertGrads, ws, stream=None):
    _check("moe_expert_ffn_backward", lib().moe_expert_ffn_backward(
        ctypes.byref(cfg), _p(x_perm), _p(x), _p(offsets), ctypes.byref(weights), _p(dy_perm), _p(dy), _p(dx_perm),
        _p(dx_shared), ctypes.byref(grads), _p(ws), _nbytes(ws), _s(stream)))


def moe_expert_ffn_backward_saved(cfg, x_perm, x, offsets, weights: MoeExpertWeights, saved: MoeFfnSaved, dy_perm,
                                  dy, dx_perm, dx_shared, grads: MoeExpertGrads, ws, stream=None):
    _check("moe_expert_ffn_backward_saved", lib().moe_expert_ffn_backward_saved(
        ctypes.byref(cfg), _p(x_perm), _p(x), _p(offsets), ctypes.byref(weights), ctypes.byref(saved), _p(dy_perm),
        _p(dy), _p(dx_perm), _p(dx_shared), ctypes.byref(grads), _p(ws), _nbytes(ws), _s(stream)))


def moe_route_backward(cfg, x, w_router, scores, topk_idx, d_topk_w, alpha, seq_len, dx_router, dw_router, loss, ws,
                       stream=None):
    _check("moe_route_backward", lib().moe_route_backward(
        ctypes.byref(cfg), _p(x), _p(w_router), _p(scores), _p(topk_idx), _p(d_topk_w), float(alpha), int(seq_len),
        _p(dx_router), _p(dw_router), _p(loss), _p(ws), _nbytes(ws), _s(stream)))


def moe_dispatch_backward(cfg, dx_perm, dx_shared, dx_router, inv, dx, stream=None):
    _check("moe_dispatch_backward", lib().moe_dispatch_backward(
        ctypes.byref(cfg), _p(dx_perm), _p(dx_shared), _p(dx_router), _p(inv), _p(dx), _s(stream)))


def moe_update_bias(cfg, counts, bias, gamma, stream=None):
    _check("moe_update_bias", lib().moe_update_bias(ctypes.byref(cfg), _p(counts), _p(bias), float(gamma),
                                                    _s(stream)))


def moe_quantize_fp8(src, n_mat, rows, cols, block_rows, dst, scales, stream=None):
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(_p(src), n_mat, rows, cols, block_rows, _p(dst),
                                                      _p(scales), _s(stream)))


def moe_ffn_workspace_part(cfg, part) -> tuple:
    """(byte offset, byte size) of an intermediate inside the moe_expert_ffn workspace."""
    off, nb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("moe_ffn_workspace_part", lib().moe_ffn_workspace_part(ctypes.byref(cfg), part, ctypes.byref(off),
                                                                  ctypes.byref(nb)))
    return int(off.value), int(nb.value)


def moe_workspace_bytes(cfg, which) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(cfg), which))


def status_string(st: int) -> str:
    try:
        return lib().moe_status_string(st).decode()
    except Exception:  # pragma: no cover
        return "?"


moe_status_string = status_string


def moe_abi_version() -> int:
    return int(lib().moe_abi_version())
