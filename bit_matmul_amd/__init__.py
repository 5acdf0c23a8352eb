"""Python binding of liblq, the MI355X (gfx950) LiftQuant decode operator.

Thin argument marshalling over the C ABI of include/lq.h: each function has
the name of the C entry point it calls, takes torch tensors that live on the
GPU (used only as device memory) plus the sizes, and enqueues on the current
torch stream unless a stream handle is given. Every step of the computation
runs in the library's HIP kernels; if liblq.so is missing, importing this
package fails.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (LQ_MULTI_MAX, LQ_ENCODE_MAX_D, LQ_ENCODE_MAX_SMALL_D, LQ_ENCODE_PINV_MAX_D,
                   LQ_ENCODE_PINV_MAX_FREE, LQ_ALGO_AUTO, LQ_ALGO_FUSED, LQ_ALGO_FUSED_LOCAL, LQ_ALGO_MFMA_LARGE, LQ_ALGO_WSPACE, LQ_ALGO_FUSED_SPLIT,
                   LQ_ALGO_MFMA_SMALL,
                   LQ_ALGO_VALU, LQ_BF16, LQ_F32, LQ_MAX_D, LQ_MAX_HB, LQ_WS_CONTROL_BYTES,
                   LQ_WS_ERROR_WORD, LQ_NOALLOC_SCRATCH_BYTES, LQ_ERR_DEVICE, LQ_MAX_L, LQError,
                   LQLayer, LQPlanInfo)

__all__ = [
    "lq_version", "lq_packed_size", "lq_pack_signs", "lq_unpack_signs", "lq_hadamard_scale",
    "lq_lift_activations", "lq_sign_gemm_workspace_size", "lq_sign_gemm", "lq_sign_gemm_ex",
    "lq_linear_workspace_size", "lq_linear", "lq_linear_workspace_size_ex", "lq_linear_ex",
    "lq_linear_algo", "lq_linear_multi_workspace_size", "lq_linear_multi", "LQ_MULTI_MAX",
    "lq_encode", "lq_train_m_step_workspace_size", "lq_train_m_step",
    "LQ_ENCODE_MAX_D", "LQ_ENCODE_MAX_SMALL_D", "LQ_ENCODE_PINV_MAX_D", "LQ_ENCODE_PINV_MAX_FREE",
    "lq_encode_pinv_workspace_size", "lq_encode_pinv",
    "lq_workspace_init", "lq_profile_events", "layer_struct", "LQError", "LQLayer",
    "LQ_F32", "LQ_BF16", "LQ_ALGO_AUTO", "LQ_ALGO_VALU", "LQ_ALGO_MFMA_SMALL",
    "LQ_ALGO_MFMA_LARGE", "LQ_ALGO_FUSED", "LQ_ALGO_FUSED_LOCAL", "LQ_ALGO_WSPACE", "LQ_ALGO_FUSED_SPLIT", "LQ_MAX_D", "LQ_MAX_HB", "LQ_WS_CONTROL_BYTES",
    "LQ_WS_ERROR_WORD", "library_path", "lq_linear_noalloc", "LQ_NOALLOC_SCRATCH_BYTES",
    "lq_linear_plan", "lq_sign_gemm_plan", "lq_workspace_status", "lq_debug_fused_timeout",
    "LQ_ERR_DEVICE", "LQ_MAX_L", "LQPlanInfo",
]

_DTYPES = {torch.float32: LQ_F32, torch.bfloat16: LQ_BF16}


def library_path() -> str:
    return str(_lib.LIB_PATH)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LQError(status, where)


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t.data_ptr()


def _opt(t, name):
    return None if t is None else _dev(t, name)


def _dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"{name} must be float32 or bfloat16")
    return _DTYPES[t.dtype]


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def lq_version() -> int:
    return _lib.LIB.lq_version()


def lq_packed_size(N: int, K: int, d: int, D: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.LIB.lq_packed_size(N, K, d, D, ctypes.byref(out)), "lq_packed_size")
    return out.value


def lq_pack_signs(signs, N, K, d, D, packed, stream=None) -> None:
    _check(_lib.LIB.lq_pack_signs(_dev(signs, "signs"), N, K, d, D, _dev(packed, "packed"),
                                  _stream(stream)), "lq_pack_signs")


def lq_unpack_signs(packed, N, K, d, D, signs, stream=None) -> None:
    _check(_lib.LIB.lq_unpack_signs(_dev(packed, "packed"), N, K, d, D, _dev(signs, "signs"),
                                    _stream(stream)), "lq_unpack_signs")


def lq_hadamard_scale(x, B, K, hb, c, xt, stream=None) -> None:
    _check(_lib.LIB.lq_hadamard_scale(_dev(x, "x"), _dtype(x, "x"), B, K, hb, _dev(c, "c"),
                                      _dev(xt, "xt"), _stream(stream)), "lq_hadamard_scale")


def lq_lift_activations(xt, B, K, d, D, M, z, stream=None) -> None:
    _check(_lib.LIB.lq_lift_activations(_dev(xt, "xt"), B, K, d, D, _dev(M, "M"), _dev(z, "z"),
                                        _dtype(z, "z"), _stream(stream)), "lq_lift_activations")


def lq_sign_gemm_workspace_size(B, N, L, ztype, algo=LQ_ALGO_AUTO) -> int:
    out = ctypes.c_size_t()
    zt = _DTYPES[ztype] if isinstance(ztype, torch.dtype) else int(ztype)
    _check(_lib.LIB.lq_sign_gemm_workspace_size(B, N, L, zt, algo, ctypes.byref(out)),
           "lq_sign_gemm_workspace_size")
    return out.value


def lq_sign_gemm_ex(packed, z, B, N, L, row_scale, y, algo, ws=None, stream=None) -> None:
    ws_ptr = _opt(ws, "ws")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.LIB.lq_sign_gemm_ex(_dev(packed, "packed"), _dev(z, "z"), _dtype(z, "z"), B, N, L,
                                    _dev(row_scale, "row_scale"), _dev(y, "y"), _dtype(y, "y"),
                                    algo, ws_ptr, ws_bytes, _stream(stream)), "lq_sign_gemm_ex")


def lq_sign_gemm(packed, z, B, N, L, row_scale, y, ws=None, stream=None) -> None:
    ws_ptr = _opt(ws, "ws")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.LIB.lq_sign_gemm(_dev(packed, "packed"), _dev(z, "z"), _dtype(z, "z"), B, N, L,
                                 _dev(row_scale, "row_scale"), _dev(y, "y"), _dtype(y, "y"),
                                 ws_ptr, ws_bytes, _stream(stream)), "lq_sign_gemm")


def layer_struct(N, K, d, D, hb, packed, M, c, row_scale) -> LQLayer:
    """Fill a ``struct lq_layer`` from device tensors (the caller keeps the
    tensors alive while the struct is used)."""
    return LQLayer(N, K, d, D, hb, 0, _dev(packed, "packed"), _dev(M, "M"), _dev(c, "c"),
                   _dev(row_scale, "row_scale"))


def lq_linear_workspace_size(layer: LQLayer, B, xtype) -> int:
    out = ctypes.c_size_t()
    xt = _DTYPES[xtype] if isinstance(xtype, torch.dtype) else int(xtype)
    _check(_lib.LIB.lq_linear_workspace_size(ctypes.byref(layer), B, xt, ctypes.byref(out)),
           "lq_linear_workspace_size")
    return out.value


def lq_linear(layer: LQLayer, x, B, y, ws=None, stream=None) -> None:
    ws_ptr = _opt(ws, "ws")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.LIB.lq_linear(ctypes.byref(layer), _dev(x, "x"), _dtype(x, "x"), B, _dev(y, "y"),
                              _dtype(y, "y"), ws_ptr, ws_bytes, _stream(stream)), "lq_linear")


def lq_linear_noalloc(layer: LQLayer, x, B, y, stream=None) -> None:
    """lq_linear with the library's own device scratch (no workspace)."""
    _check(_lib.LIB.lq_linear_noalloc(ctypes.byref(layer), _dev(x, "x"), _dtype(x, "x"), B,
                                      _dev(y, "y"), _dtype(y, "y"), _stream(stream)),
           "lq_linear_noalloc")


def lq_linear_workspace_size_ex(layer: LQLayer, B, xtype, algo) -> int:
    out = ctypes.c_size_t()
    xt = _DTYPES[xtype] if isinstance(xtype, torch.dtype) else int(xtype)
    _check(_lib.LIB.lq_linear_workspace_size_ex(ctypes.byref(layer), B, xt, algo, ctypes.byref(out)),
           "lq_linear_workspace_size_ex")
    return out.value


def lq_linear_algo(layer: LQLayer, B, xtype, algo=0) -> int:
    """The algorithm lq_linear_ex runs for these arguments (AUTO resolved)."""
    out = ctypes.c_int()
    xt = _DTYPES[xtype] if isinstance(xtype, torch.dtype) else int(xtype)
    _check(_lib.LIB.lq_linear_algo(ctypes.byref(layer), B, xt, algo, ctypes.byref(out)),
           "lq_linear_algo")
    return out.value


def lq_linear_plan(layer: LQLayer, B, xtype, algo=LQ_ALGO_AUTO) -> dict:
    """Algorithm and sign-product launch shape lq_linear_ex would use."""
    info = LQPlanInfo()
    xt = _DTYPES[xtype] if isinstance(xtype, torch.dtype) else int(xtype)
    _check(_lib.LIB.lq_linear_plan(ctypes.byref(layer), B, xt, algo, ctypes.byref(info)),
           "lq_linear_plan")
    return {f: getattr(info, f) for f, _ in LQPlanInfo._fields_}


def lq_sign_gemm_plan(B, N, L, ztype, algo=LQ_ALGO_AUTO) -> dict:
    """Algorithm and launch shape lq_sign_gemm_ex would use."""
    info = LQPlanInfo()
    zt = _DTYPES[ztype] if isinstance(ztype, torch.dtype) else int(ztype)
    _check(_lib.LIB.lq_sign_gemm_plan(B, N, L, zt, algo, ctypes.byref(info)), "lq_sign_gemm_plan")
    return {f: getattr(info, f) for f, _ in LQPlanInfo._fields_}


def lq_workspace_status(ws, stream=None) -> int:
    """LQ_OK, or LQ_ERR_DEVICE when a call on this workspace reported a
    failure (waits for the stream). Other errors raise."""
    st = _lib.LIB.lq_workspace_status(_dev(ws, "ws"), ws.numel() * ws.element_size(),
                                      _stream(stream))
    if st not in (0, LQ_ERR_DEVICE):
        _check(st, "lq_workspace_status")
    return st


def lq_debug_fused_timeout(enable: bool) -> None:
    _check(_lib.LIB.lq_debug_fused_timeout(1 if enable else 0), "lq_debug_fused_timeout")


def lq_linear_ex(layer: LQLayer, x, B, y, algo, ws=None, stream=None) -> None:
    ws_ptr = _opt(ws, "ws")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.LIB.lq_linear_ex(ctypes.byref(layer), _dev(x, "x"), _dtype(x, "x"), B, _dev(y, "y"),
                                 _dtype(y, "y"), algo, ws_ptr, ws_bytes, _stream(stream)),
           "lq_linear_ex")


def _layer_array(layers):
    arr = (LQLayer * len(layers))()
    for i, l in enumerate(layers):
        arr[i] = l
    return arr


def lq_linear_multi_workspace_size(layers, B, xtype) -> int:
    """Workspace bytes of lq_linear_multi for these layers (same K)."""
    out = ctypes.c_size_t()
    xt = _DTYPES[xtype] if isinstance(xtype, torch.dtype) else int(xtype)
    arr = _layer_array(layers)
    _check(_lib.LIB.lq_linear_multi_workspace_size(arr, len(layers), B, xt, ctypes.byref(out)),
           "lq_linear_multi_workspace_size")
    return out.value


def lq_linear_multi(layers, x, B, ys, ws=None, stream=None) -> None:
    """ys[i] = lq_linear(layers[i], x) for every layer (same K, same x, one
    y dtype): one preparation and one product launch where that applies."""
    if len(ys) != len(layers):
        raise ValueError("one output per layer")
    ws_ptr = _opt(ws, "ws")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    ydt = _dtype(ys[0], "y")
    for y in ys:
        if _dtype(y, "y") != ydt:
            raise ValueError("every output must have the same dtype")
    ptrs = (ctypes.c_void_p * len(ys))(*[_dev(y, "y") for y in ys])
    arr = _layer_array(layers)
    _check(_lib.LIB.lq_linear_multi(arr, len(layers), _dev(x, "x"), _dtype(x, "x"), B, ptrs, ydt,
                                    ws_ptr, ws_bytes, _stream(stream)), "lq_linear_multi")


def lq_encode(w, nblocks, d, D, M, signs, dist2=None, stream=None) -> None:
    """Nearest-neighbour encoding: signs[b] = argmin_s ||w_b - M s|| (float32
    w, M; int8 signs; optional float32 squared distances)."""
    for t, name, dt in ((w, "w", torch.float32), (M, "M", torch.float32), (signs, "signs", torch.int8)):
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt}")
    if dist2 is not None and dist2.dtype != torch.float32:
        raise ValueError("dist2 must be float32")
    _check(_lib.LIB.lq_encode(_dev(w, "w"), nblocks, d, D, _dev(M, "M"), _dev(signs, "signs"),
                              _opt(dist2, "dist2"), _stream(stream)), "lq_encode")


def lq_encode_pinv_workspace_size(d, D) -> int:
    out = ctypes.c_size_t()
    _check(_lib.LIB.lq_encode_pinv_workspace_size(d, D, ctypes.byref(out)),
           "lq_encode_pinv_workspace_size")
    return out.value


def lq_encode_pinv(w, nblocks, d, D, M, signs, dist2=None, ws=None, stream=None) -> None:
    """The 2^(D-d) pseudo-inverse-initialised search (float32 w, M; int8
    signs; optional float32 squared distances; ws: uint8 device tensor of
    lq_encode_pinv_workspace_size bytes)."""
    for t, name, dt in ((w, "w", torch.float32), (M, "M", torch.float32), (signs, "signs", torch.int8)):
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt}")
    if dist2 is not None and dist2.dtype != torch.float32:
        raise ValueError("dist2 must be float32")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.LIB.lq_encode_pinv(_dev(w, "w"), nblocks, d, D, _dev(M, "M"), _dev(signs, "signs"),
                                   _opt(dist2, "dist2"), _opt(ws, "ws"), ws_bytes, _stream(stream)),
           "lq_encode_pinv")


def lq_train_m_step_workspace_size(n, d, D) -> int:
    out = ctypes.c_size_t()
    _check(_lib.LIB.lq_train_m_step_workspace_size(n, d, D, ctypes.byref(out)),
           "lq_train_m_step_workspace_size")
    return out.value


def lq_train_m_step(M, w, n, d, D, lr, loss=None, ws=None, stream=None) -> None:
    """One gradient step of Eq. (1) on M (float32, updated in place) over the
    samples w (n x d float32); loss (one float32) receives the loss at the
    old M."""
    if M.dtype != torch.float32 or w.dtype != torch.float32:
        raise ValueError("M and w must be float32")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.LIB.lq_train_m_step(_dev(M, "M"), _dev(w, "w"), n, d, D, float(lr),
                                    _opt(loss, "loss"), _opt(ws, "ws"), ws_bytes, _stream(stream)),
           "lq_train_m_step")


def lq_workspace_init(ws, stream=None) -> None:
    """Zero the control area of a workspace before its first use."""
    _check(_lib.LIB.lq_workspace_init(_dev(ws, "ws"), ws.numel() * ws.element_size(),
                                      _stream(stream)), "lq_workspace_init")


def lq_profile_events(starts, stops) -> None:
    """Bracket every sign-product kernel launch with the given hipEvent_t
    handles (sequences of ints, used round-robin); empty sequences clear it."""
    n = len(starts)
    if len(stops) != n:
        raise ValueError("starts and stops must have the same length")
    arr = ctypes.c_void_p * max(n, 1)
    _check(_lib.LIB.lq_profile_events(arr(*starts), arr(*stops), n), "lq_profile_events")
