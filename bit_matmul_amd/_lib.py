"""ctypes loader and prototypes for liblq.so (the C ABI in include/lq.h)."""
from __future__ import annotations

import ctypes
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "liblq.so"

LQ_OK, LQ_ERR_INVALID_ARG, LQ_ERR_UNSUPPORTED, LQ_ERR_WORKSPACE, LQ_ERR_HIP, LQ_ERR_DEVICE = range(6)
LQ_F32, LQ_BF16 = 0, 1
(LQ_ALGO_AUTO, LQ_ALGO_VALU, LQ_ALGO_MFMA_SMALL, LQ_ALGO_MFMA_LARGE, LQ_ALGO_FUSED,
 LQ_ALGO_FUSED_LOCAL, LQ_ALGO_WSPACE, LQ_ALGO_FUSED_SPLIT) = range(8)
LQ_MAX_D = 64
LQ_MAX_HB = 1024
LQ_MAX_L = 1 << 28
LQ_WS_CONTROL_BYTES = 20992
LQ_WS_ERROR_WORD = 96
LQ_ENCODE_MAX_D = 24
LQ_ENCODE_MAX_SMALL_D = 16
LQ_ENCODE_PINV_MAX_D = 32
LQ_ENCODE_PINV_MAX_FREE = 24
LQ_MULTI_MAX = 4
LQ_NOALLOC_SCRATCH_BYTES = 16 << 20

# Every symbol include/lq.h declares.
EXPORTS = [
    "lq_version", "lq_status_string", "lq_last_hip_error", "lq_packed_size",
    "lq_pack_signs", "lq_unpack_signs", "lq_hadamard_scale", "lq_lift_activations",
    "lq_sign_gemm_workspace_size", "lq_sign_gemm", "lq_sign_gemm_ex",
    "lq_linear_workspace_size", "lq_linear", "lq_linear_workspace_size_ex", "lq_linear_ex",
    "lq_linear_algo", "lq_workspace_init", "lq_profile_events", "lq_encode",
    "lq_train_m_step_workspace_size", "lq_train_m_step", "lq_linear_multi_workspace_size",
    "lq_linear_multi", "lq_linear_noalloc", "lq_linear_plan", "lq_sign_gemm_plan",
    "lq_workspace_status", "lq_debug_fused_timeout", "lq_encode_pinv_workspace_size",
    "lq_encode_pinv",
]


class LQLayer(ctypes.Structure):
    """Mirror of ``struct lq_layer``."""
    _fields_ = [
        ("N", c_int64), ("K", c_int64), ("d", c_int32), ("D", c_int32),
        ("hb", c_int32), ("reserved", c_int32),
        ("packed", c_void_p), ("M", c_void_p), ("c", c_void_p), ("row_scale", c_void_p),
    ]


class LQPlanInfo(ctypes.Structure):
    """Mirror of ``struct lq_plan_info``."""
    _fields_ = [
        ("algo", c_int32), ("workgroups", c_int32), ("waves", c_int32), ("panels", c_int32),
        ("batch_rows", c_int32), ("ksplit", c_int32),
    ]


class LQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = LIB.lq_status_string(status).decode() if LIB is not None else str(status)
        if status == LQ_ERR_HIP and LIB is not None:
            msg += f" (hipError {LIB.lq_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def _load():
    if not LIB_PATH.exists():
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m bit_matmul_amd.build` "
            "(the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(str(LIB_PATH))
    i64, i32, sz, vp = c_int64, c_int32, c_size_t, c_void_p
    protos = {
        "lq_version": (c_int, []),
        "lq_status_string": (c_char_p, [c_int]),
        "lq_last_hip_error": (c_int, []),
        "lq_packed_size": (c_int, [i64, i64, i32, i32, POINTER(sz)]),
        "lq_pack_signs": (c_int, [vp, i64, i64, i32, i32, vp, vp]),
        "lq_unpack_signs": (c_int, [vp, i64, i64, i32, i32, vp, vp]),
        "lq_hadamard_scale": (c_int, [vp, c_int, i64, i64, i32, vp, vp, vp]),
        "lq_lift_activations": (c_int, [vp, i64, i64, i32, i32, vp, vp, c_int, vp]),
        "lq_sign_gemm_workspace_size": (c_int, [i64, i64, i64, c_int, c_int, POINTER(sz)]),
        "lq_sign_gemm": (c_int, [vp, vp, c_int, i64, i64, i64, vp, vp, c_int, vp, sz, vp]),
        "lq_sign_gemm_ex": (c_int, [vp, vp, c_int, i64, i64, i64, vp, vp, c_int, c_int, vp, sz, vp]),
        "lq_linear_workspace_size": (c_int, [POINTER(LQLayer), i64, c_int, POINTER(sz)]),
        "lq_linear": (c_int, [POINTER(LQLayer), vp, c_int, i64, vp, c_int, vp, sz, vp]),
        "lq_linear_workspace_size_ex": (c_int, [POINTER(LQLayer), i64, c_int, c_int, POINTER(sz)]),
        "lq_linear_algo": (c_int, [POINTER(LQLayer), i64, c_int, c_int, POINTER(c_int)]),
        "lq_encode": (c_int, [vp, i64, c_int32, c_int32, vp, vp, vp, vp]),
        "lq_encode_pinv_workspace_size": (c_int, [c_int32, c_int32, POINTER(sz)]),
        "lq_encode_pinv": (c_int, [vp, i64, c_int32, c_int32, vp, vp, vp, vp, sz, vp]),
        "lq_train_m_step_workspace_size": (c_int, [i64, c_int32, c_int32, POINTER(sz)]),
        "lq_train_m_step": (c_int, [vp, vp, i64, c_int32, c_int32, c_float, vp, vp, sz, vp]),
        "lq_linear_ex": (c_int, [POINTER(LQLayer), vp, c_int, i64, vp, c_int, c_int, vp, sz, vp]),
        "lq_linear_multi_workspace_size": (c_int, [POINTER(LQLayer), c_int32, i64, c_int,
                                                   POINTER(sz)]),
        "lq_linear_multi": (c_int, [POINTER(LQLayer), c_int32, vp, c_int, i64, POINTER(vp), c_int,
                                    vp, sz, vp]),
        "lq_linear_noalloc": (c_int, [POINTER(LQLayer), vp, c_int, i64, vp, c_int, vp]),
        "lq_workspace_init": (c_int, [vp, sz, vp]),
        "lq_linear_plan": (c_int, [POINTER(LQLayer), i64, c_int, c_int, POINTER(LQPlanInfo)]),
        "lq_sign_gemm_plan": (c_int, [i64, i64, i64, c_int, c_int, POINTER(LQPlanInfo)]),
        "lq_workspace_status": (c_int, [vp, sz, vp]),
        "lq_debug_fused_timeout": (c_int, [i32]),
        "lq_profile_events": (c_int, [POINTER(vp), POINTER(vp), i32]),
    }
    for name, (res, args) in protos.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()
