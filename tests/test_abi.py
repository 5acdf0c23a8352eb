"""The C ABI without a GPU: the library loads, exports every declared symbol,
computes storage sizes, and rejects invalid calls before enqueueing anything.

Pointer arguments here are fake (aligned integers that are never
dereferenced): each call is chosen so that host-side validation rejects it,
or so that it is an empty call that returns without touching the device.
"""
import ctypes
import re
from pathlib import Path

import pytest

from bit_matmul_amd import _lib
from bit_matmul_amd._lib import (LIB, LQ_BF16, LQ_ERR_INVALID_ARG, LQ_ERR_UNSUPPORTED,
                                 LQ_ERR_WORKSPACE, LQ_F32, LQ_OK, LQLayer)
from oracle import liftquant_ref as ref
from workloads import WORKLOADS

HEADER = Path(__file__).resolve().parent.parent / "include" / "lq.h"
P = 0x100000            # fake, 16-byte aligned device address (never dereferenced)
MIS = P + 4             # misaligned


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(LIB, n), f"liblq.so does not export {n}"
    assert sorted(_lib.EXPORTS) == names


def test_version_and_status_strings():
    assert LIB.lq_version() == 100
    for s in range(5):
        assert LIB.lq_status_string(s).decode().startswith("LQ_")
    assert LIB.lq_last_hip_error() == 0


def size(N, K, d, D):
    out = ctypes.c_size_t()
    st = LIB.lq_packed_size(N, K, d, D, ctypes.byref(out))
    return st, out.value


def test_packed_size_matches_storage_formula():
    for wl in WORKLOADS.values():
        for l in wl.layers:
            st, b = size(l.N, l.K, l.d, l.D)
            assert st == LQ_OK
            assert b * 8 == ref.packed_bits(l.N, l.K, l.d, l.D)
    # values quoted for the Llama-3-8B gate/up and the 70B QKV shapes
    assert size(14336, 4096, 10, 24) == (LQ_OK, 17633280)
    assert size(10240, 8192, 10, 24) == (LQ_OK, 25190400)


@pytest.mark.parametrize("args,status", [
    ((-16, 64, 2, 5), LQ_ERR_INVALID_ARG),
    ((16, 0, 2, 5), LQ_ERR_INVALID_ARG),
    ((16, 64, 0, 5), LQ_ERR_INVALID_ARG),
    ((16, 64, 6, 5), LQ_ERR_INVALID_ARG),       # D < d
    ((16, 64, 2, 65), LQ_ERR_UNSUPPORTED),      # D > LQ_MAX_D
    ((15, 64, 2, 8), LQ_ERR_UNSUPPORTED),       # N % 16
    ((16, 6, 2, 5), LQ_ERR_UNSUPPORTED),        # L = 15, not a multiple of 8
])
def test_packed_size_rejects(args, status):
    assert size(*args)[0] == status


def test_packed_size_null_output():
    assert LIB.lq_packed_size(16, 64, 2, 8, None) == LQ_ERR_INVALID_ARG


def test_pack_validation():
    f = LIB.lq_pack_signs
    assert f(None, 16, 64, 2, 8, P, None) == LQ_ERR_INVALID_ARG
    assert f(P, 16, 64, 2, 8, MIS, None) == LQ_ERR_INVALID_ARG
    assert f(P, 17, 64, 2, 8, P, None) == LQ_ERR_UNSUPPORTED
    assert f(P, 0, 64, 2, 8, P, None) == LQ_OK                # empty: nothing enqueued
    assert LIB.lq_unpack_signs(None, 16, 64, 2, 8, P, None) == LQ_ERR_INVALID_ARG


def test_hadamard_validation():
    f = LIB.lq_hadamard_scale
    assert f(P, LQ_F32, 1, 96, 3, P, P, None) == LQ_ERR_INVALID_ARG     # hb not a power of 2
    assert f(P, LQ_F32, 1, 4096, 2048, P, P, None) == LQ_ERR_UNSUPPORTED
    assert f(P, LQ_F32, 1, 96, 64, P, P, None) == LQ_ERR_INVALID_ARG    # hb does not divide K
    assert f(P, 7, 1, 64, 64, P, P, None) == LQ_ERR_INVALID_ARG         # bad dtype
    assert f(MIS, LQ_F32, 1, 64, 64, P, P, None) == LQ_ERR_INVALID_ARG
    assert f(P, LQ_F32, 1, 64, 64, None, P, None) == LQ_ERR_INVALID_ARG
    assert f(P, LQ_F32, -1, 64, 64, P, P, None) == LQ_ERR_INVALID_ARG
    assert f(P, LQ_F32, 0, 64, 64, P, P, None) == LQ_OK


def test_lift_validation():
    f = LIB.lq_lift_activations
    assert f(P, 1, 64, 5, 2, P, P, LQ_F32, None) == LQ_ERR_INVALID_ARG   # D < d
    assert f(P, 1, 64, 2, 100, P, P, LQ_F32, None) == LQ_ERR_UNSUPPORTED
    assert f(P, 1, 64, 2, 5, None, P, LQ_F32, None) == LQ_ERR_INVALID_ARG
    assert f(P, 1, 64, 2, 5, P, P, 3, None) == LQ_ERR_INVALID_ARG
    assert f(P, 0, 64, 2, 5, P, P, LQ_BF16, None) == LQ_OK


def ws_size(B, N, L, zt, algo):
    out = ctypes.c_size_t()
    st = LIB.lq_sign_gemm_workspace_size(B, N, L, zt, algo, ctypes.byref(out))
    return st, out.value


def test_sign_gemm_validation_and_workspace():
    f = LIB.lq_sign_gemm_ex
    st, need = ws_size(1, 4096, 34416, LQ_F32, 1)
    assert st == LQ_OK and need > 0
    st3, need3 = ws_size(1, 4096, 34416, LQ_BF16, 3)
    assert st3 == LQ_OK and need3 >= 34416 * 16 * 2     # z in operand order: 16 rows per tile
    assert ws_size(17, 4096, 34416, LQ_BF16, 2)[0] == LQ_ERR_UNSUPPORTED   # small MFMA: B <= 16
    assert ws_size(1, 4096, 34416, LQ_BF16, 9)[0] == LQ_ERR_INVALID_ARG
    assert ws_size(1, 4095, 34416, LQ_BF16, 0)[0] == LQ_ERR_UNSUPPORTED
    assert ws_size(1, 4096, 34415, LQ_BF16, 0)[0] == LQ_ERR_UNSUPPORTED
    # too small / missing workspace
    assert f(P, P, LQ_F32, 1, 4096, 34416, P, P, LQ_F32, 1, P, need - 1, None) == LQ_ERR_WORKSPACE
    assert f(P, P, LQ_F32, 1, 4096, 34416, P, P, LQ_F32, 1, None, 0, None) == LQ_ERR_WORKSPACE
    # misaligned / null operands
    assert f(MIS, P, LQ_F32, 1, 4096, 34416, P, P, LQ_F32, 1, P, need, None) == LQ_ERR_INVALID_ARG
    assert f(P, P, LQ_F32, 1, 4096, 34416, None, P, LQ_F32, 1, P, need, None) == LQ_ERR_INVALID_ARG
    assert f(P, P, LQ_F32, 1, 4096, 34416, P, P, 5, 1, P, need, None) == LQ_ERR_INVALID_ARG
    # empty batch: valid, enqueues nothing
    assert f(None, None, LQ_F32, 0, 4096, 34416, None, None, LQ_F32, 0, None, 0, None) == LQ_OK


def test_linear_validation():
    lay = LQLayer(4096, 14336, 10, 24, 1024, 0, P, P, P, P)
    out = ctypes.c_size_t()
    assert LIB.lq_linear_workspace_size(ctypes.byref(lay), 1, LQ_BF16, ctypes.byref(out)) == LQ_OK
    need = out.value
    assert need >= 34416 * 12 // 8    # at least two 6-bit terms per lifted column
    f = LIB.lq_linear
    assert f(ctypes.byref(lay), P, LQ_BF16, 1, P, LQ_BF16, P, need - 1, None) == LQ_ERR_WORKSPACE
    bad = LQLayer(4096, 14336, 10, 24, 1000, 0, P, P, P, P)
    assert f(ctypes.byref(bad), P, LQ_BF16, 1, P, LQ_BF16, P, need, None) == LQ_ERR_INVALID_ARG
    bad = LQLayer(4096, 14336, 10, 24, 1024, 1, P, P, P, P)       # reserved != 0
    assert f(ctypes.byref(bad), P, LQ_BF16, 1, P, LQ_BF16, P, need, None) == LQ_ERR_INVALID_ARG
    bad = LQLayer(4096, 14336, 10, 24, 1024, 0, P, MIS, P, P)
    assert f(ctypes.byref(bad), P, LQ_BF16, 1, P, LQ_BF16, P, need, None) == LQ_ERR_INVALID_ARG
    assert f(None, P, LQ_BF16, 1, P, LQ_BF16, P, need, None) == LQ_ERR_INVALID_ARG
    assert f(ctypes.byref(lay), P, LQ_BF16, 0, P, LQ_BF16, None, 0, None) == LQ_OK


def linear_ws_size(lay, B, xt, algo):
    out = ctypes.c_size_t()
    st = LIB.lq_linear_workspace_size_ex(ctypes.byref(lay), B, xt, algo, ctypes.byref(out))
    return st, out.value


def test_linear_ex_validation_and_control_area():
    lay = LQLayer(4096, 14336, 10, 24, 1024, 0, P, P, P, P)
    for algo in (0, 1, 2, 3):
        st, need = linear_ws_size(lay, 1, LQ_BF16, algo)
        assert st == LQ_OK
        # every workspace that is used at all starts with the control area
        assert need >= _lib.LQ_WS_CONTROL_BYTES + 34416 * 3 // 4
    assert linear_ws_size(lay, 1, LQ_BF16, 8)[0] == LQ_ERR_INVALID_ARG
    # one launch split over the reduction: batch 1, a partial per tile group
    gate7 = LQLayer(14336, 4096, 10, 24, 1024, 0, P, P, P, P)
    st, need7 = linear_ws_size(gate7, 1, LQ_BF16, 7)
    assert st == LQ_OK and need7 >= _lib.LQ_WS_CONTROL_BYTES + 14336 * 4
    assert linear_ws_size(lay, 1, LQ_BF16, 7)[0] == LQ_OK                   # down, K = 14336
    assert linear_ws_size(lay, 2, LQ_BF16, 7)[0] == LQ_ERR_UNSUPPORTED     # batch 1 only
    assert ws_size(1, 4096, 34416, LQ_BF16, 7)[0] == LQ_ERR_INVALID_ARG    # sign_gemm: no
    # W space: D in {4, 8}, d <= 4, bf16 x, any batch
    assert linear_ws_size(lay, 1, LQ_BF16, 6)[0] == LQ_ERR_UNSUPPORTED       # D = 24
    pre = LQLayer(8192, 8192, 3, 8, 1024, 0, P, P, P, P)
    st, need = linear_ws_size(pre, 2048, LQ_BF16, 6)
    L = 2731 * 8
    tiles = -(-L // 512)
    assert st == LQ_OK
    assert need >= (_lib.LQ_WS_CONTROL_BYTES
                    + 128 * 2 * tiles * 3 * 1024                          # xp: d KB per step
                    + 512 * 1024)                                         # tail slots
    assert need < _lib.LQ_WS_CONTROL_BYTES + 2048 * 8192 * 4               # no fp32 xt
    assert linear_ws_size(pre, 2048, LQ_F32, 6)[0] == LQ_ERR_UNSUPPORTED    # fp32 x
    assert linear_ws_size(LQLayer(8192, 8192, 5, 8, 1024, 0, P, P, P, P), 64, LQ_BF16, 6)[0] \
        == LQ_ERR_UNSUPPORTED                                                # d > 4
    assert linear_ws_size(LQLayer(4096, 512, 2, 4, 512, 0, P, P, P, P), 3, LQ_BF16, 6)[0] == LQ_OK
    assert ws_size(64, 8192, L, LQ_BF16, 6)[0] == LQ_ERR_INVALID_ARG       # sign_gemm: no W space
    # one launch without communication: batch 1, rows up to 8192, no workspace
    assert linear_ws_size(lay, 1, LQ_BF16, 5)[0] == LQ_ERR_UNSUPPORTED       # K = 14336
    gate = LQLayer(14336, 4096, 10, 24, 1024, 0, P, P, P, P)
    assert linear_ws_size(gate, 1, LQ_BF16, 5) == (LQ_OK, 0)
    assert linear_ws_size(gate, 2, LQ_BF16, 5)[0] == LQ_ERR_UNSUPPORTED
    assert linear_ws_size(lay, 17, LQ_BF16, 4)[0] == LQ_ERR_UNSUPPORTED      # one launch: B <= 16
    assert linear_ws_size(lay, 8, LQ_BF16, 4)[0] == LQ_ERR_UNSUPPORTED       # 24 operand columns
    assert linear_ws_size(lay, 17, LQ_BF16, 1)[0] == LQ_ERR_UNSUPPORTED      # VALU linear: B <= 16
    assert ws_size(1, 4096, 34416, LQ_BF16, 4)[0] == LQ_ERR_INVALID_ARG      # sign_gemm: no FUSED
    assert linear_ws_size(lay, 0, LQ_BF16, 4) == (LQ_OK, 0)
    f = LIB.lq_linear_ex
    need = linear_ws_size(lay, 1, LQ_BF16, 2)[1]
    assert f(ctypes.byref(lay), P, LQ_BF16, 1, P, LQ_BF16, 2, P, need - 1, None) == LQ_ERR_WORKSPACE
    assert f(ctypes.byref(lay), P, LQ_BF16, 1, P, LQ_BF16, 8, P, need, None) == LQ_ERR_INVALID_ARG
    assert f(ctypes.byref(lay), P, LQ_BF16, 1, P, LQ_BF16, 6, P, need, None) == LQ_ERR_UNSUPPORTED
    assert f(ctypes.byref(lay), P, LQ_BF16, 17, P, LQ_BF16, 4, P, need, None) == LQ_ERR_UNSUPPORTED
    assert f(ctypes.byref(lay), P, LQ_BF16, 0, P, LQ_BF16, 4, None, 0, None) == LQ_OK


def test_workspace_init_validation():
    f = LIB.lq_workspace_init
    assert f(None, 0, None) == LQ_OK
    assert f(P, 0, None) == LQ_OK
    assert f(None, 64, None) == LQ_ERR_INVALID_ARG
    assert f(MIS, 64, None) == LQ_ERR_INVALID_ARG


def test_profile_events_validation():
    f = LIB.lq_profile_events
    arr = (ctypes.c_void_p * 2)(P, P)
    assert f(None, None, -1) == LQ_ERR_INVALID_ARG
    assert f(None, arr, 2) == LQ_ERR_INVALID_ARG
    nulls = (ctypes.c_void_p * 2)(P, None)
    assert f(arr, nulls, 2) == LQ_ERR_INVALID_ARG
    assert f(None, None, 0) == LQ_OK


def test_linear_algo_resolution():
    f = LIB.lq_linear_algo
    out = ctypes.c_int(-1)

    def res(lay, B, xt, algo=0):
        st = f(ctypes.byref(lay), B, xt, algo, ctypes.byref(out))
        return st, out.value
    gate = LQLayer(14336, 4096, 10, 24, 1024, 0, P, P, P, P)
    pre = LQLayer(8192, 8192, 3, 8, 1024, 0, P, P, P, P)
    qwen = LQLayer(27648, 5120, 2, 5, 1024, 0, P, P, P, P)
    assert res(gate, 1, LQ_BF16) == (LQ_OK, 2)        # MFMA_SMALL
    assert res(gate, 1, 0) == (LQ_OK, 1)              # fp32 x: VALU
    assert res(pre, 2048, LQ_BF16) == (LQ_OK, 6)      # W space
    assert res(pre, 2048, 0) == (LQ_OK, 3)            # fp32 x: lifted MFMA
    assert res(qwen, 64, LQ_BF16) == (LQ_OK, 3)       # D = 5: lifted MFMA
    assert res(pre, 2048, LQ_BF16, 3) == (LQ_OK, 3)   # explicit choice kept
    assert res(gate, 2, LQ_BF16, 5)[0] == LQ_ERR_UNSUPPORTED
    assert res(gate, 0, LQ_BF16)[0] == LQ_ERR_INVALID_ARG
    assert f(ctypes.byref(gate), 1, LQ_BF16, 0, None) == LQ_ERR_INVALID_ARG
    assert res(gate, 1, LQ_BF16, 8)[0] == LQ_ERR_INVALID_ARG
    assert res(gate, 1, LQ_BF16, 7) == (LQ_OK, 7)


def test_encode_and_train_validation():
    f = LIB.lq_encode
    assert f(P, 0, 3, 8, P, P, None, None) == LQ_OK                     # nothing to do
    assert f(None, 4, 3, 8, P, P, None, None) == LQ_ERR_INVALID_ARG
    assert f(P, 4, 3, 8, None, P, None, None) == LQ_ERR_INVALID_ARG
    assert f(P, 4, 3, 8, P, None, None, None) == LQ_ERR_INVALID_ARG
    assert f(P, -1, 3, 8, P, P, None, None) == LQ_ERR_INVALID_ARG
    assert f(P, 4, 9, 8, P, P, None, None) == LQ_ERR_INVALID_ARG       # d > D
    assert f(P, 4, 0, 8, P, P, None, None) == LQ_ERR_INVALID_ARG
    assert f(P, 4, 3, 25, P, P, None, None) == LQ_ERR_UNSUPPORTED      # 2^25 per block
    assert f(P, 4, 17, 24, P, P, None, None) == LQ_ERR_UNSUPPORTED     # d > 16
    odd = P + 2
    assert f(odd, 4, 3, 8, P, P, None, None) == LQ_ERR_INVALID_ARG
    assert f(P, 4, 3, 8, P, P, odd, None) == LQ_ERR_INVALID_ARG
    out = ctypes.c_size_t()
    g = LIB.lq_train_m_step_workspace_size
    assert g(1000, 3, 8, ctypes.byref(out)) == LQ_OK
    assert out.value >= 1000 * 8 + 4 * (3 * 8 + 1) * 8                 # signs + partials
    assert g(0, 3, 8, ctypes.byref(out)) == LQ_OK and out.value == 0
    assert g(10, 3, 8, None) == LQ_ERR_INVALID_ARG
    assert g(10, 3, 30, ctypes.byref(out)) == LQ_ERR_UNSUPPORTED
    t = LIB.lq_train_m_step
    need = 1000 * 8 + 4 * (3 * 8 + 1) * 8
    assert t(P, P, 1000, 3, 8, ctypes.c_float(0.1), None, P, 16, None) == LQ_ERR_WORKSPACE
    assert t(P, P, 1000, 3, 8, ctypes.c_float(0.1), None, None, 0, None) == LQ_ERR_WORKSPACE
    assert t(None, P, 1000, 3, 8, ctypes.c_float(0.1), None, P, need, None) == LQ_ERR_INVALID_ARG
    assert t(P, P, 0, 3, 8, ctypes.c_float(0.1), None, None, 0, None) == LQ_OK


def test_encode_pinv_validation():
    f = LIB.lq_encode_pinv
    g = LIB.lq_encode_pinv_workspace_size
    out = ctypes.c_size_t()
    assert g(16, 32, ctypes.byref(out)) == LQ_OK and out.value == 16 * 32 * 8   # M_a^-1, M_a^-1 M_f
    assert g(3, 8, ctypes.byref(out)) == LQ_OK and out.value == 256              # (192 rounded up)
    assert g(3, 8, None) == LQ_ERR_INVALID_ARG
    assert g(3, 33, ctypes.byref(out)) == LQ_ERR_UNSUPPORTED                     # D > 32
    assert g(2, 27, ctypes.byref(out)) == LQ_ERR_UNSUPPORTED                     # 2^25 per block
    assert g(17, 32, ctypes.byref(out)) == LQ_ERR_UNSUPPORTED                    # d > 16
    assert g(9, 8, ctypes.byref(out)) == LQ_ERR_INVALID_ARG                      # d > D
    ws = 4096
    assert f(P, 0, 16, 32, P, P, None, None, 0, None) == LQ_OK                   # nothing to do
    assert f(None, 4, 16, 32, P, P, None, P, ws, None) == LQ_ERR_INVALID_ARG
    assert f(P, 4, 16, 32, None, P, None, P, ws, None) == LQ_ERR_INVALID_ARG
    assert f(P, 4, 16, 32, P, None, None, P, ws, None) == LQ_ERR_INVALID_ARG
    assert f(P, -1, 16, 32, P, P, None, P, ws, None) == LQ_ERR_INVALID_ARG
    assert f(P, 4, 16, 32, P, P, None, None, 0, None) == LQ_ERR_WORKSPACE
    assert f(P, 4, 16, 32, P, P, None, P, ws - 1, None) == LQ_ERR_WORKSPACE
    assert f(P, 4, 16, 32, P, P, None, P + 8, ws, None) == LQ_ERR_INVALID_ARG    # ws not 16-aligned
    assert f(P, 4, 2, 27, P, P, None, P, ws, None) == LQ_ERR_UNSUPPORTED
    assert f(P + 2, 4, 16, 32, P, P, None, P, ws, None) == LQ_ERR_INVALID_ARG   # w not 4-aligned


def multi_ws_size(layers, B, xt, n=None):
    arr = (LQLayer * max(1, len(layers)))(*layers)
    out = ctypes.c_size_t()
    st = LIB.lq_linear_multi_workspace_size(arr, len(layers) if n is None else n, B, xt,
                                            ctypes.byref(out))
    return st, out.value


def test_linear_multi_plan_and_validation():
    gate = LQLayer(14336, 4096, 10, 24, 1024, 0, P, P, P, P)
    down = LQLayer(4096, 14336, 10, 24, 1024, 0, P, P, P, P)
    st, one = linear_ws_size(gate, 1, LQ_BF16, 0)
    assert st == LQ_OK
    # grouped (bf16 x, batch 1): the control area, one operand per layer (20
    # records of 896 bytes: two terms of one batch row, and 1 KB of slack)
    # and the partial row sums of the layers whose rows are split into
    # reduction ranges
    operand = 20 * 896 + 1024
    st, two = multi_ws_size([gate, gate], 1, LQ_BF16)
    assert st == LQ_OK
    assert _lib.LQ_WS_CONTROL_BYTES + 2 * operand <= two <= _lib.LQ_WS_CONTROL_BYTES + 2 * (one - _lib.LQ_WS_CONTROL_BYTES)
    st, four = multi_ws_size([gate] * 4, 1, LQ_BF16)
    assert st == LQ_OK and four >= _lib.LQ_WS_CONTROL_BYTES + 4 * operand
    # fp32 x and large batches run the layers one after another: one call's workspace
    assert multi_ws_size([gate, gate], 1, LQ_F32) == linear_ws_size(gate, 1, LQ_F32, 0)
    assert multi_ws_size([gate, gate], 64, LQ_BF16) == linear_ws_size(gate, 64, LQ_BF16, 0)
    # one layer: as lq_linear
    assert multi_ws_size([gate], 1, LQ_BF16) == (LQ_OK, one)
    # errors: layers of different K, no layers, too many, bad layer, NULL outputs
    assert multi_ws_size([gate, down], 1, LQ_BF16)[0] == LQ_ERR_INVALID_ARG
    assert multi_ws_size([gate], 1, LQ_BF16, n=0)[0] == LQ_ERR_INVALID_ARG
    assert multi_ws_size([gate] * 5, 1, LQ_BF16)[0] == LQ_ERR_INVALID_ARG
    bad = LQLayer(14336, 4096, 10, 24, 1000, 0, P, P, P, P)              # hb not a power of 2
    assert multi_ws_size([gate, bad], 1, LQ_BF16)[0] == LQ_ERR_INVALID_ARG
    arr = (LQLayer * 2)(gate, gate)
    assert LIB.lq_linear_multi(arr, 2, P, LQ_BF16, 1, None, LQ_BF16, P, two, None) == LQ_ERR_INVALID_ARG
    ys = (ctypes.c_void_p * 2)(P, P)
    assert LIB.lq_linear_multi(arr, 2, P, LQ_BF16, 1, ys, LQ_BF16, P, two - 16, None) == LQ_ERR_WORKSPACE
    assert LIB.lq_linear_multi(arr, 2, P, LQ_BF16, 0, ys, LQ_BF16, None, 0, None) == LQ_OK   # B = 0


# ------------------------------------------------------------ plan queries

from tests.plan_cases import LARGE_PLAN_CASES, LARGE_SPLIT_CASES, case_id, split_case_id  # noqa: E402


@pytest.mark.parametrize("case", LARGE_PLAN_CASES, ids=[case_id(c) for c in LARGE_PLAN_CASES])
def test_large_batch_plan_of_each_parity_shape(case):
    """Each shape of the large-batch parity tests selects the tiling it is
    listed for, so every instantiated tiling is compared with the oracle."""
    N, L, B, zt, pw, jb = case
    info = _lib.LQPlanInfo()
    st = LIB.lq_sign_gemm_plan(B, N, L, LQ_BF16 if zt == "bf16" else LQ_F32, 3, ctypes.byref(info))
    assert st == LQ_OK
    assert info.algo == 3 and info.waves == 4
    assert (info.panels // 4, info.batch_rows // 16) == (pw, jb)
    assert info.ksplit == 1
    assert info.workgroups == -(-N // (16 * 4 * pw)) * -(-(-(-B // 16)) // jb)


@pytest.mark.parametrize("case", LARGE_SPLIT_CASES, ids=[split_case_id(c) for c in LARGE_SPLIT_CASES])
def test_large_batch_plan_splits_the_reduction(case):
    """Too few panel and batch groups for the chip: reduction ranges of >= 8
    tiles, as many as keep the workgroups within 512, none empty."""
    N, L, B, zt, pw, jb, ks = case
    info = _lib.LQPlanInfo()
    zdt = LQ_BF16 if zt == "bf16" else LQ_F32
    assert LIB.lq_sign_gemm_plan(B, N, L, zdt, 3, ctypes.byref(info)) == LQ_OK
    assert (info.panels // 4, info.batch_rows // 16, info.ksplit) == (pw, jb, ks)
    groups = -(-N // (16 * 4 * pw)) * -(-(-(-B // 16)) // jb)
    assert info.workgroups == groups * ks and info.workgroups <= 512
    ext = -(-L // 512)
    tps = -(-ext // ks)
    assert tps >= 8 and (ks - 1) * tps < ext
    # the workspace holds the operand in product order and the fp32 partial
    # sums of every range
    size = ctypes.c_size_t()
    assert LIB.lq_sign_gemm_workspace_size(B, N, L, zdt, 3, ctypes.byref(size)) == LQ_OK
    nterm = 1 if zt == "bf16" else 2
    zp = nterm * -(-B // 16) * 4 * ext * 4096
    assert size.value >= zp + ks * B * N * 4


def test_linear_plan_of_the_benchmarked_layers():
    """lq_linear's choice on the workloads: the small-batch matrix-core
    product at B <= 16 (bf16 x), W space for the prefill layers, the lifted
    large-batch product for the Qwen layers at B = 64."""
    info = _lib.LQPlanInfo()
    for wl in WORKLOADS.values():
        for s in wl.layers:
            lay = LQLayer(s.N, s.K, s.d, s.D, s.hb, 0, P, P, P, P)
            for B in wl.batches:
                xt = LQ_F32 if wl.xdtype == "f32" else LQ_BF16
                assert LIB.lq_linear_plan(ctypes.byref(lay), B, xt, 0, ctypes.byref(info)) == LQ_OK
                if B > 16:
                    want = 6 if s.D in (4, 8) and s.d <= 4 else 3
                else:
                    want = 1 if xt == LQ_F32 else 2
                assert info.algo == want, (wl.name, s.name, B)
                assert info.workgroups > 0 and info.waves > 0 and info.panels > 0
                if want == 6 and B >= 2048:
                    # 4 panels per wavefront, 8 batch tiles per workgroup
                    assert (info.panels, info.batch_rows) == (16, 128), (s.name, B)
                if want == 3 and B == 64:
                    # 2 panels per wavefront, 4 batch tiles, the reduction
                    # split so that every compute unit has a workgroup
                    ks = {"up": 2, "down": 12}[s.name]
                    assert (info.panels, info.batch_rows, info.ksplit) == (8, 64, ks), s.name
                    assert info.workgroups >= 256
    assert LIB.lq_linear_plan(None, 1, LQ_BF16, 0, ctypes.byref(info)) == LQ_ERR_INVALID_ARG
    lay = LQLayer(16, 64, 2, 8, 64, 0, P, P, P, P)
    assert LIB.lq_linear_plan(ctypes.byref(lay), 0, LQ_BF16, 0, ctypes.byref(info)) == LQ_ERR_INVALID_ARG
    assert LIB.lq_linear_plan(ctypes.byref(lay), 1, LQ_BF16, 0, None) == LQ_ERR_INVALID_ARG


def test_chunked_plan_counts_loader_wavefronts():
    """The 70B down projection at B = 4 and 16 (bf16 x) runs the chunked
    small-batch product: its records neither fit LDS nor stream. The plan
    reports the launch's wavefronts: the compute ones (8 with one column set
    of 16 (batch row, term) columns, 4 with two) and the four loaders."""
    info = _lib.LQPlanInfo()
    lay = LQLayer(8192, 28672, 10, 24, 1024, 0, P, P, P, P)
    for B, waves in ((4, 8 + 4), (16, 4 + 4)):
        assert LIB.lq_linear_plan(ctypes.byref(lay), B, LQ_BF16, 0, ctypes.byref(info)) == LQ_OK
        assert info.algo == 2 and info.panels == 2 and info.workgroups == 256
        assert info.waves == waves, (B, info.waves)


def test_lifted_length_cap():
    """L above LQ_MAX_L (2^28 lifted columns per row) is rejected: byte
    offsets inside a panel (2 L) then stay within 32 bits."""
    assert size(16, 1 << 28, 1, 1)[0] == LQ_OK
    assert size(16, (1 << 28) + 8, 1, 1)[0] == LQ_ERR_UNSUPPORTED
    out = ctypes.c_size_t()
    assert LIB.lq_sign_gemm_workspace_size(1, 16, (1 << 28) + 8, LQ_BF16, 0,
                                           ctypes.byref(out)) == LQ_ERR_UNSUPPORTED


def test_device_status_code_and_short_workspace_status():
    assert LIB.lq_status_string(5).decode().startswith("LQ_ERR_DEVICE")
    # a workspace without a control area cannot hold a failure: no device access
    assert LIB.lq_workspace_status(P, 16, None) == LQ_OK
    assert LIB.lq_workspace_status(None, 0, None) == LQ_OK
    assert LIB.lq_workspace_status(MIS, 1 << 20, None) == LQ_ERR_INVALID_ARG
