"""CPU oracle of the LiftQuant lift-then-project decode operator.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

Everything is plain numpy in float64, written for readability, not speed.

Sources, cited by title and section:

* [paper] "LiftQuant: Continuous Bit-Width LLM via Dimensional Lifting and
  Projection" (arXiv 2606.04050), read in its Chinese translation
  ("LiftQuant：基于维度提升与投影的连续比特宽度大语言模型量化框架").
* [review] "Paper Review: LiftQuant: Continuous Bit-Width LLM via Dimensional
  Lifting and Projection" (romaanj.github.io), the "Method" paragraph.

What the operator computes, in the pages' notation:

* A length-d weight block is stored as D signs w_q in {+1,-1}^D and decoded as
  w = M w_q with one d x D mapping matrix M ([paper] §3.1; [review] Method).
  The effective bit-width is D/d ([paper] §3 introduction; Fig. 2).
* The fused decode operator is o = diag(s) W (M T a) ([paper] §3 introduction;
  [review] Method: diag(s) W_q (T* a^T), an INT1 x FP GEMM plus small linear
  maps). T is a layer-wise whitening: Hadamard mixing plus per-channel scaling
  ([paper] §3 introduction, forward reference to §3.2; [review] Method).
* Written out, o is the plain linear map y = diag(s) W_dense (T a), with
  W_dense assembled block by block from w = M w_q. This oracle computes that
  plain definition; the lifted route S (M^T T a) is the same map rearranged and
  is provided separately (``lift`` and ``sign_matmul``) for the kernels that
  compute the individual steps.

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):

* T = blockdiag_q(H_hb diag(c_q)) with H_hb the orthonormal Hadamard matrix in
  Sylvester order, H[i, j] = (-1)^popcount(i & j) / sqrt(hb): scale each
  channel, then mix each hb-block. T itself is not learned here.
* K is zero-padded to K' = d * ceil(K / d) after T, before the lift.
* Lifted column j of a row is j = b * D + e for block b and sign e.
* The row scale is called ``row_scale`` (the paper's diag(s)); ``signs`` are
  the w_q.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "hadamard", "whitening_block", "whiten", "pad_blocks", "decode_weight",
    "linear", "lift", "sign_matmul", "packed_bits", "bits_per_weight",
    "codebook", "sign_pattern", "encode_nn", "encode_pinv", "train_m_step", "orthonormal_rows",
]


def _popcount(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.int64)
    count = np.zeros_like(a)
    while np.any(a):
        count += a & 1
        a >>= 1
    return count


def hadamard(hb: int) -> np.ndarray:
    """Orthonormal Hadamard matrix of order ``hb`` (a power of two), Sylvester
    order: H[i, j] = (-1)^popcount(i & j) / sqrt(hb).

    The channel mixing of the whitening transform starts from a Hadamard
    matrix ([paper] §3 introduction; [review] Method). Order and normalisation
    are not given on the pages; this is the reading taken.
    """
    if hb < 1 or hb & (hb - 1):
        raise ValueError("Hadamard order must be a power of two")
    i = np.arange(hb)
    parity = _popcount(i[:, None] & i[None, :]) % 2
    return np.where(parity == 0, 1.0, -1.0) / np.sqrt(hb)


def whitening_block(c_block: np.ndarray) -> np.ndarray:
    """One diagonal block of T: T_q = H_hb diag(c_q), as an explicit dense
    hb x hb matrix: per-channel scaling followed by orthogonal mixing
    ([paper] §3 introduction; [review] Method)."""
    c_block = np.asarray(c_block, dtype=np.float64)
    return hadamard(len(c_block)) @ np.diag(c_block)


def whiten(x: np.ndarray, c: np.ndarray, hb: int) -> np.ndarray:
    """xt = T x for every batch row: T is block diagonal with blocks
    H_hb diag(c_q), one per consecutive run of hb channels.

    x: (B, K); c: (K,); hb must divide K. Returns (B, K) float64.
    """
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    B, K = x.shape
    if K % hb:
        raise ValueError("hb must divide K")
    xt = np.empty_like(x)
    for q in range(K // hb):
        sl = slice(q * hb, (q + 1) * hb)
        Tq = whitening_block(c[sl])
        xt[:, sl] = x[:, sl] @ Tq.T          # each row: Tq @ x_row
    return xt


def pad_blocks(xt: np.ndarray, d: int) -> np.ndarray:
    """Append zero columns so the width becomes a multiple of the block
    length d (K' = d * ceil(K / d))."""
    xt = np.asarray(xt, dtype=np.float64)
    B, K = xt.shape
    Kp = -(-K // d) * d
    out = np.zeros((B, Kp))
    out[:, :K] = xt
    return out


def decode_weight(signs: np.ndarray, M: np.ndarray) -> np.ndarray:
    """Dense weight rows from lifted signs: block b of row n is
    w = M w_q with w_q = signs[n, b, :] ([paper] §3.1, definition of the
    mapping matrix; [review] Method).

    signs: (N, Kb, D) with entries +1/-1; M: (d, D). Returns (N, Kb * d).
    """
    signs = np.asarray(signs)
    M = np.asarray(M, dtype=np.float64)
    N, Kb, D = signs.shape
    d = M.shape[0]
    if M.shape[1] != D:
        raise ValueError("M must be d x D")
    W = np.empty((N, Kb * d))
    for b in range(Kb):
        s_b = signs[:, b, :].astype(np.float64)      # (N, D), one w_q per row
        W[:, b * d:(b + 1) * d] = s_b @ M.T          # row n: M @ s_b[n]
    return W


def linear(x: np.ndarray, c: np.ndarray, hb: int, M: np.ndarray,
           signs: np.ndarray, row_scale: np.ndarray) -> np.ndarray:
    """The decode operator o = diag(s) W (T a) for a batch of activations
    ([paper] §3 introduction, fused operator; [review] Method).

    x: (B, K) activations; c: (K,) channel scales of T; hb: Hadamard block;
    M: (d, D); signs: (N, Kb, D); row_scale: (N,). Returns y: (B, N) float64
    with y[b, n] = row_scale[n] * sum_k W[n, k] * xt_pad[b, k].
    """
    d = np.asarray(M).shape[0]
    xt = pad_blocks(whiten(x, c, hb), d)
    W = decode_weight(signs, M)
    if W.shape[1] != xt.shape[1]:
        raise ValueError("signs do not match ceil(K/d) blocks")
    y = xt @ W.T
    return y * np.asarray(row_scale, dtype=np.float64)[None, :]


def lift(xt_pad: np.ndarray, M: np.ndarray) -> np.ndarray:
    """Lifted activations: z_b = M^T xt_b for each length-d block b, laid out
    as z[:, b * D + e]. This is the M T a factor of the fused operator
    ([paper] §3 introduction), written T* a^T in [review] Method.

    xt_pad: (B, Kb * d); M: (d, D). Returns (B, Kb * D).
    """
    xt_pad = np.asarray(xt_pad, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    d, D = M.shape
    B, Kp = xt_pad.shape
    if Kp % d:
        raise ValueError("width must be a multiple of d")
    Kb = Kp // d
    z = np.empty((B, Kb * D))
    for b in range(Kb):
        z[:, b * D:(b + 1) * D] = xt_pad[:, b * d:(b + 1) * d] @ M
    return z


def sign_matmul(signs_flat: np.ndarray, z: np.ndarray,
                row_scale: np.ndarray) -> np.ndarray:
    """The INT1 x FP product of the decode path with its row scale:
    y = diag(s) W_q z ([review] Method; [paper] §3 introduction).

    signs_flat: (N, L) +1/-1; z: (B, L); row_scale: (N,). Returns (B, N).
    """
    S = np.asarray(signs_flat).astype(np.float64)
    z = np.asarray(z, dtype=np.float64)
    return (z @ S.T) * np.asarray(row_scale, dtype=np.float64)[None, :]


def packed_bits(N: int, K: int, d: int, D: int) -> int:
    """Storage of one quantized layer in bits: every one of the N rows holds
    ceil(K / d) blocks of D one-bit signs ([paper] §3 introduction and §3.1)."""
    return N * (-(-K // d)) * D


def bits_per_weight(K: int, d: int, D: int) -> float:
    """Effective bits per original weight, D/d when d divides K ([paper] §3
    introduction; Fig. 2)."""
    return (-(-K // d)) * D / K


def sign_pattern(index: int, D: int) -> np.ndarray:
    """The sign vector numbered ``index``: s_e = -1 when bit e of index is set."""
    return np.array([-1.0 if (index >> e) & 1 else 1.0 for e in range(D)])


def codebook(M: np.ndarray) -> np.ndarray:
    """All 2^D codewords M s, s in {+1,-1}^D, in the order of ``sign_pattern``
    (the implicit codebook of [paper] §3.1 and Fig. 2). Returns (2^D, d)."""
    M = np.asarray(M, dtype=np.float64)
    D = M.shape[1]
    return np.stack([M @ sign_pattern(i, D) for i in range(1 << D)])


def encode_nn(w: np.ndarray, M: np.ndarray):
    """Nearest-neighbour encoding of d-blocks: for every row w_b of w (n x d),
    the sign vector s in {+1,-1}^D whose codeword M s is closest to w_b in
    Euclidean distance. This is the inner minimisation of [paper] §3.1
    Eq. (1), which the paper names the nearest-neighbour search, i.e. the
    quantization step. Exhaustive over the 2^D sign vectors, numbered as in
    ``sign_pattern`` and visited in that order (in chunks, to bound memory);
    among equally close codewords the lowest number wins.

    Returns (signs (n, D) of +-1, squared distances (n,))."""
    M = np.asarray(M, dtype=np.float64)
    d, D = M.shape
    w = np.asarray(w, dtype=np.float64).reshape(-1, d)
    n = w.shape[0]
    best = np.full(n, np.inf)
    idx = np.zeros(n, dtype=np.int64)
    chunk = 1 << min(D, 16)
    for p0 in range(0, 1 << D, chunk):
        numbers = np.arange(p0, p0 + chunk, dtype=np.int64)
        S = np.where((numbers[:, None] >> np.arange(D)[None, :]) & 1, -1.0, 1.0)   # sign_pattern rows
        cw = S @ M.T                                                               # codewords M s
        for a in range(0, n, 64):
            diff = w[a:a + 64, None, :] - cw[None, :, :]
            dist = (diff * diff).sum(axis=2)                                       # (<=64, chunk)
            i = np.argmin(dist, axis=1)                                            # first minimum
            v = dist[np.arange(i.size), i]
            take = v < best[a:a + 64]                                              # strictly closer only
            best[a:a + 64] = np.where(take, v, best[a:a + 64])
            idx[a:a + 64] = np.where(take, p0 + i, idx[a:a + 64])
    signs = np.where((idx[:, None] >> np.arange(D)[None, :]) & 1, -1.0, 1.0)
    return signs, best


def encode_pinv(w: np.ndarray, M: np.ndarray):
    """The nearest-neighbour search reduced from 2^D to 2^(D-d) sign vectors by
    pseudo-inverse initialisation ([review] Method: "accelerated from 2^D to
    2^(D-d) by pseudo-inverse initialization"; [review] Limitations: the exact
    search is practically capped at D - d <= 20). The pages give no more; the
    reading taken here:

    * M = [M_a | M_f]: the first d columns M_a (d x d) are solved for, the
      other D - d columns M_f are enumerated.
    * For each of the 2^(D-d) sign vectors s_f of the enumerated columns, the
      solved signs are the signs of the pseudo-inverse solution
      u = pinv(M_a) (w - M_f s_f) (the least-squares lifted coordinates given
      s_f), s_a = sgn(u) with sgn(0) = +1; the candidate is s = (s_a, s_f).
    * The candidate closest to w in Euclidean distance wins; among equally
      close ones, the lowest pattern index (bit e set meaning s_e = -1, as in
      ``sign_pattern``).

    Where M_a is diagonal (a multiple of the identity in particular) the
    minimisation over s_a separates per coordinate and sgn(u) is its exact
    minimiser, so the result is the exhaustive search's (``encode_nn``); in
    general it visits a subset of the sign vectors, so its distance is never
    below the exhaustive one.

    Returns (signs (n, D) of +-1, squared distances (n,))."""
    M = np.asarray(M, dtype=np.float64)
    d, D = M.shape
    F = D - d
    w = np.asarray(w, dtype=np.float64).reshape(-1, d)
    n = w.shape[0]
    Ma, Mf = M[:, :d], M[:, d:]
    A = np.linalg.pinv(Ma)
    q = np.arange(1 << F, dtype=np.int64)                                   # free-sign patterns
    Sf = np.where((q[:, None] >> np.arange(F)[None, :]) & 1, -1.0, 1.0)    # (2^F, F)
    signs = np.zeros((n, D))
    best = np.zeros(n)
    for b in range(n):
        U = (A @ (w[b][:, None] - Mf @ Sf.T)).T                             # (2^F, d): pinv(M_a)(w - M_f s_f)
        Sa = np.where(U >= 0.0, 1.0, -1.0)
        R = w[b][None, :] - Sa @ Ma.T - Sf @ Mf.T                           # w - M s
        dist = (R * R).sum(axis=1)
        idx = ((Sa < 0) * (1 << np.arange(d))[None, :]).sum(axis=1) + (q << d)
        k = np.lexsort((idx, dist))[0]                                      # least distance, then index
        signs[b, :d], signs[b, d:] = Sa[k], Sf[k]
        best[b] = dist[k]
    return signs, best


def orthonormal_rows(G: np.ndarray, d: int) -> np.ndarray:
    """A d x D matrix with orthonormal rows, from a D x D Gaussian draw G: the
    first d columns of the Q factor of G, transposed ([paper] §3.1 "Optimising
    M": the rows of M are initialised as orthonormal vectors)."""
    q, r = np.linalg.qr(np.asarray(G, dtype=np.float64))
    q = q * np.sign(np.diag(r))[None, :]               # the unique Q with diag(R) > 0
    return q[:, :d].T.copy()


def train_m_step(M: np.ndarray, w: np.ndarray, lr: float):
    """One gradient step on the objective of [paper] §3.1 Eq. (1) estimated on
    the samples w (n x d, drawn from N(0, I_d)):

        loss(M) = mean_b min_s || w_b - M s ||      (the norm as printed)

    The minimiser s_b* is piecewise constant in M, so wherever it is unique
    the gradient of the minimum is the gradient of || w_b - M s_b* || with
    s_b* held fixed (Danskin's theorem): -(r_b / ||r_b||) s_b*^T with
    r_b = w_b - M s_b* (zero where r_b = 0). Plain gradient descent:
    M <- M - lr * mean_b of that gradient.

    Returns (the updated M, the loss at the old M)."""
    M = np.asarray(M, dtype=np.float64)
    d, D = M.shape
    w = np.asarray(w, dtype=np.float64).reshape(-1, d)
    signs, _ = encode_nn(w, M)
    r = w - signs @ M.T                                # (n, d) residuals
    norm = np.sqrt((r * r).sum(axis=1))
    loss = float(norm.mean()) if norm.size else 0.0
    unit = np.where(norm[:, None] > 0, r / np.where(norm > 0, norm, 1.0)[:, None], 0.0)
    grad = -(unit.T @ signs) / max(1, w.shape[0])      # d x D
    return M - lr * grad, loss

