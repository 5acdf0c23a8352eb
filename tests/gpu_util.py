"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the library through its C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda"


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so a crash still shows it)."""
    sys.stdout.write(f"\n[gpu] {msg}\n")
    sys.stdout.flush()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t if dtype is None else t.to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


class DeviceLayer:
    """A layer's tensors on the GPU, packed by lq_pack_signs."""

    def __init__(self, li, lq):
        s = li.spec
        self.spec = s
        self.N, self.K, self.d, self.D, self.hb, self.L = s.N, s.K, s.d, s.D, s.hb, s.L
        signs = dev(li.signs().reshape(s.N, s.L))
        self.packed = torch.empty(lq.lq_packed_size(s.N, s.K, s.d, s.D), dtype=torch.uint8, device=DEV)
        note(f"lq_pack_signs N={s.N} K={s.K} d={s.d} D={s.D}")
        lq.lq_pack_signs(signs, s.N, s.K, s.d, s.D, self.packed)
        torch.cuda.synchronize()
        del signs
        self.M = dev(li.M)
        self.c = dev(li.c)
        self.r = dev(li.row_scale)
        self.struct = lq.layer_struct(s.N, s.K, s.d, s.D, s.hb, self.packed, self.M, self.c, self.r)

    def linear(self, lq, x: torch.Tensor, B: int, ydtype, algo=None) -> torch.Tensor:
        """lq_linear (algo None) or lq_linear_ex on a fresh workspace whose
        contents beyond the control area are garbage; checks the error word."""
        y = torch.empty((B, self.N), dtype=ydtype, device=DEV)
        a = lq.LQ_ALGO_AUTO if algo is None else algo
        nbytes = lq.lq_linear_workspace_size_ex(self.struct, B, x.dtype, a)
        ws = workspace(lq, nbytes)
        note(f"lq_linear N={self.N} K={self.K} d={self.d} D={self.D} hb={self.hb} B={B} "
             f"x={x.dtype} algo={algo}")
        if algo is None:
            lq.lq_linear(self.struct, x, B, y, ws)
        else:
            lq.lq_linear_ex(self.struct, x, B, y, algo, ws)
        torch.cuda.synchronize()
        assert control_error(lq, ws) == 0
        assert lq.lq_workspace_status(ws) == 0
        return y


def workspace(lq, nbytes: int) -> torch.Tensor:
    """A workspace with garbage contents and a zeroed control area."""
    ws = torch.full((max(nbytes, 16),), 0xA5, dtype=torch.uint8, device=DEV)
    lq.lq_workspace_init(ws)
    return ws


def control_error(lq, ws: torch.Tensor) -> int:
    if ws.numel() < lq.LQ_WS_CONTROL_BYTES:
        return 0
    return int(ws[: lq.LQ_WS_CONTROL_BYTES].view(torch.int32)[lq.LQ_WS_ERROR_WORD].item())


def sign_gemm(lq, packed, z: torch.Tensor, B, N, L, r, ydtype, algo):
    y = torch.empty((B, N), dtype=ydtype, device=DEV)
    nbytes = lq.lq_sign_gemm_workspace_size(B, N, L, z.dtype, algo)
    ws = workspace(lq, nbytes)
    note(f"lq_sign_gemm_ex algo={algo} B={B} N={N} L={L} z={z.dtype} y={ydtype}")
    lq.lq_sign_gemm_ex(packed, z, B, N, L, r, y, algo, ws)
    torch.cuda.synchronize()
    return y
