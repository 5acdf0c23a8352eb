"""Seeded draws of every input of one quantized linear layer.

Distributions (one ``numpy.random.Generator(PCG64(seed))`` stream per layer,
drawn in this fixed order so that weights are identical across batch sizes):

1. ``M``: d x D float32, entries ~ N(0, 1/D).
2. signs: N x L independent fair coin flips (L = ceil(K/d) * D), drawn as
   N*L/8 random bytes; bit e of byte t of row n is the flip of lifted column
   8*t + e, and a set bit means the sign -1.
3. ``row_scale``: N float32 ~ U[0.5, 1.5].
4. ``c``: K float32 ~ U[0.8, 1.2] (per-channel scales of the whitening).
5. outlier channels: round(frac * K) distinct channel indices.
6. ``x``: B_max x K float32 ~ N(0, 1); outlier channels multiplied by the
   gain; then rounded to bfloat16 (round-to-nearest-even) when the workload's
   activations are bf16. Smaller batches take the leading rows.

Nothing here computes any part of the operator.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import LayerSpec, Workload


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16, returned as float32."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32).reshape(np.shape(x))


def sign_bits_to_int8(sign_bytes: np.ndarray, N: int, L: int) -> np.ndarray:
    """Expand the drawn coin-flip bytes to an int8 array of +1/-1, N x L."""
    bits = np.unpackbits(sign_bytes.reshape(N, L // 8), axis=1, bitorder="little")
    out = np.ones((N, L), dtype=np.int8)
    out[bits.astype(bool)] = -1
    return out


@dataclass
class LayerInputs:
    spec: LayerSpec
    M: np.ndarray            # (d, D) float32
    sign_bytes: np.ndarray   # (N * L / 8,) uint8, raw coin flips
    row_scale: np.ndarray    # (N,) float32
    c: np.ndarray            # (K,) float32
    outliers: np.ndarray     # (n_out,) int64 channel indices
    x_max: np.ndarray        # (B_max, K) float32, dtype-rounded values
    xdtype: str

    def signs(self) -> np.ndarray:
        """int8 signs shaped (N, Kb, D)."""
        s = self.spec
        return sign_bits_to_int8(self.sign_bytes, s.N, s.L).reshape(s.N, s.Kb, s.D)

    def signs_rows(self, rows: np.ndarray) -> np.ndarray:
        """int8 signs of the listed output rows, shaped (len(rows), Kb, D)."""
        s = self.spec
        per_row = s.L // 8
        sub = self.sign_bytes.reshape(s.N, per_row)[np.asarray(rows)]
        return sign_bits_to_int8(sub.reshape(-1), len(rows), s.L).reshape(len(rows), s.Kb, s.D)

    def x(self, B: int) -> np.ndarray:
        if B > self.x_max.shape[0]:
            raise ValueError(f"batch {B} exceeds drawn batch {self.x_max.shape[0]}")
        return self.x_max[:B]

    def x_bf16_bits(self, B: int) -> np.ndarray:
        return bf16_bits(self.x(B))


def _draw(spec: LayerSpec, B_max: int, xdtype: str, outlier_frac: float,
          outlier_gain: float) -> LayerInputs:
    if (spec.N * spec.L) % 8:
        raise ValueError("N*L must be a multiple of 8 to draw whole bytes")
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    M = (rng.standard_normal((spec.d, spec.D)) / np.sqrt(spec.D)).astype(np.float32)
    sign_bytes = np.frombuffer(rng.bytes(spec.N * spec.L // 8), dtype=np.uint8).copy()
    row_scale = rng.uniform(0.5, 1.5, spec.N).astype(np.float32)
    c = rng.uniform(0.8, 1.2, spec.K).astype(np.float32)
    n_out = int(round(outlier_frac * spec.K))
    outliers = np.sort(rng.choice(spec.K, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    x = rng.standard_normal((B_max, spec.K)).astype(np.float32)
    if n_out:
        x[:, outliers] *= np.float32(outlier_gain)
    if xdtype == "bf16":
        x = bf16_round(x)
    elif xdtype != "f32":
        raise ValueError(xdtype)
    return LayerInputs(spec, M, sign_bytes, row_scale, c, outliers.astype(np.int64), x, xdtype)


def make_layer(spec: LayerSpec, wl: Workload, B_max: Optional[int] = None) -> LayerInputs:
    """Inputs of one layer of a named workload (batch up to ``B_max``,
    default the workload's largest batch)."""
    B = B_max if B_max is not None else max(wl.batches)
    return _draw(spec, B, wl.xdtype, wl.outlier_frac, wl.outlier_gain)


def make_layer_small(N: int, K: int, d: int, D: int, hb: int, seed: int,
                     B_max: int = 4, xdtype: str = "f32",
                     outlier_frac: float = 0.0, outlier_gain: float = 1.0) -> LayerInputs:
    """Inputs of an arbitrary (usually small) layer shape, same recipe."""
    spec = LayerSpec(f"n{N}k{K}d{d}D{D}", K=K, N=N, d=d, D=D, hb=hb, seed=seed)
    return _draw(spec, B_max, xdtype, outlier_frac, outlier_gain)
