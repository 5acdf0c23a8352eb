"""Reference packer for the one-bit sign matrix. TEST INFRASTRUCTURE ONLY.

The pages store the lifted signs as one bit each (INT1 / UINT1 weights of the
decode GEMM: [review] "Released resources" and Method paragraphs; [paper] §3
introduction) but give no byte layout. The layout below is this library's own
format; it is written here independently of the HIP packer, and the two are
compared bit for bit.

Sign matrix S is N x L (L = ceil(K/d) * D lifted columns, column j = b*D + e).
Requirements: N % 16 == 0 and L % 8 == 0. Total size is exactly N * L / 8
bytes, i.e. N * ceil(K/d) * D bits.

* Rows are grouped in panels of 16 (panel p = rows 16p .. 16p+15). Panel p
  occupies bytes [p * 2L, (p+1) * 2L).
* Inside a panel, the first nt = L // 512 column tiles are full tiles of
  16 rows x 512 columns, 1024 bytes each, tile q at panel offset q * 1024.
  A full tile is 64 slots of 16 bytes; slot l = 16*g + r (g in 0..3,
  r in 0..15) belongs to row 16p + r. Its 32-bit little-endian word u
  (u in 0..3, at slot offset 4u) holds columns q*512 + 128u + 32g + b in
  bit b (b in 0..31).
* The remaining w = L % 512 columns (a multiple of 8, m = w / 8 bytes per row)
  form a tail at panel offset nt * 1024, stored row by row: byte t of row r is
  at r * m + t and its bit e is column nt*512 + 8t + e.
* A set bit means the sign -1, a clear bit +1.
"""
from __future__ import annotations

import numpy as np

PANEL_ROWS = 16
TILE_COLS = 512


def check_shape(N: int, L: int) -> None:
    if N % PANEL_ROWS or L % 8 or N <= 0 or L <= 0:
        raise ValueError("packed layout needs N % 16 == 0 and L % 8 == 0")


def bit_index(n: np.ndarray, j: np.ndarray, N: int, L: int) -> np.ndarray:
    """Global bit number (8 * byte + bit) of sign (n, j), vectorised."""
    check_shape(N, L)
    n = np.asarray(n, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    p, r = n // PANEL_ROWS, n % PANEL_ROWS
    q, cc = j // TILE_COLS, j % TILE_COLS
    nt = L // TILE_COLS
    m = (L - nt * TILE_COLS) // 8
    base = p * 2 * L

    u, rem = cc // 128, cc % 128
    g, b = rem // 32, rem % 32
    slot = 16 * g + r
    full_byte = base + q * 1024 + 16 * slot + 4 * u + b // 8
    full_bit = b % 8

    t, e = cc // 8, cc % 8
    tail_byte = base + nt * 1024 + r * m + t
    tail_bit = e

    in_full = q < nt
    byte = np.where(in_full, full_byte, tail_byte)
    bit = np.where(in_full, full_bit, tail_bit)
    return byte * 8 + bit


def packed_bytes(N: int, L: int) -> int:
    check_shape(N, L)
    return N * L // 8


def refpack(signs_flat: np.ndarray) -> np.ndarray:
    """Pack an N x L array of +1/-1 (any integer or float type) into the
    layout above. Returns uint8 of N * L / 8 bytes."""
    S = np.asarray(signs_flat)
    N, L = S.shape
    nn, jj = np.meshgrid(np.arange(N), np.arange(L), indexing="ij")
    idx = bit_index(nn.ravel(), jj.ravel(), N, L)
    flat = np.zeros(N * L, dtype=np.uint8)
    flat[idx] = (S.ravel() < 0).astype(np.uint8)
    return np.packbits(flat, bitorder="little")


def refunpack(packed: np.ndarray, N: int, L: int) -> np.ndarray:
    """Inverse of ``refpack``: int8 +1/-1 array of shape (N, L)."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.size != packed_bytes(N, L):
        raise ValueError("packed buffer has the wrong size")
    flat = np.unpackbits(packed, bitorder="little")
    nn, jj = np.meshgrid(np.arange(N), np.arange(L), indexing="ij")
    neg = flat[bit_index(nn.ravel(), jj.ravel(), N, L)].reshape(N, L)
    return np.where(neg == 1, -1, 1).astype(np.int8)


def refpack_panel(signs_panel: np.ndarray, L: int) -> np.ndarray:
    """Bytes of one 16-row panel (the layout is panel-local)."""
    return refpack(np.asarray(signs_panel).reshape(PANEL_ROWS, L))
