"""Checks that tie the CPU oracle to facts other than itself.

Each ``pin_*`` takes the oracle module (and the reference packer) and raises
AssertionError (or any exception) when the oracle is wrong. They are collected
by ``tests/test_oracle.py`` against the real oracle, and by
``tests/test_oracle_mutants.py`` against copies of the oracle with planted
mistakes, each of which must fail at least one pin.

What pins what:

* Hadamard matrix: scipy's Sylvester construction (a library routine), the
  Kronecker recursion and orthogonality.
* Whitening T: its action on unit vectors in closed form (T e_i = c_i H e_i),
  norm preservation when c = 1, and the diagonal case hb = 1.
* Decoding w = M w_q: exact brute force over every codeword for the four
  (D, d) cases of the paper's codeword-generation figure, with dyadic
  entries so float64 is exact; the codebook's mean and second moment in closed
  form (E[s] = 0, E[s s^T] = I so E[(Ms)(Ms)^T] = M M^T); the D = d, M = I
  special case, which reduces to a plain integer matrix product.
* The lifted route S (M^T T x) against the dense route W (T x).
* Row scale, zero padding and storage size (the pages' worked bit-widths).
* Nearest-neighbour encoding: a pure-Python loop over every sign vector
  (itertools, no codebook helper); the M = I case in closed form
  (s = sign(w), sign(0) = +1); odd symmetry and scale invariance.
* Training step of Eq. (1): central finite differences of the loss (the
  gradient of a minimum is the gradient at its minimiser), descent on the
  same samples, and orthonormal rows of the initial M.
"""
from __future__ import annotations

import itertools
from fractions import Fraction
from pathlib import Path

import numpy as np
import scipy.linalg

GOLDEN = Path(__file__).resolve().parent / "golden"


def _dyadic(rng, shape, denom=8, lim=8):
    """Random dyadic rationals k/denom, |k| <= lim, as float64 (exact)."""
    return rng.integers(-lim, lim + 1, size=shape).astype(np.float64) / denom


def _frac(a):
    return Fraction(float(a)).limit_denominator(1 << 20)


def _signs(rng, *shape):
    return np.where(rng.random(shape) < 0.5, -1, 1).astype(np.int8)


# --------------------------------------------------------------------- Hadamard

def pin_hadamard_library(o, rp=None):
    for n in [1, 2, 4, 8, 16, 64, 256, 512, 1024]:
        H = o.hadamard(n)
        ref = scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n)
        assert np.array_equal(H, ref), f"Hadamard order {n} differs from scipy"


def pin_hadamard_structure(o, rp=None):
    for n in [2, 8, 128]:
        H = o.hadamard(n)
        assert np.allclose(H @ H.T, np.eye(n), atol=1e-12)
        Hh = o.hadamard(n // 2) * np.sqrt(n // 2)
        rec = np.block([[Hh, Hh], [Hh, -Hh]]) / np.sqrt(n)
        assert np.allclose(H, rec, atol=1e-15)


# -------------------------------------------------------------------- whitening

def pin_whiten_unit_vectors(o, rp=None):
    rng = np.random.default_rng(7)
    K, hb = 32, 8
    c = rng.uniform(0.8, 1.2, K)
    xt = o.whiten(np.eye(K), c, hb)          # row i is T e_i
    Hs = scipy.linalg.hadamard(hb).astype(np.float64) / np.sqrt(hb)
    for i in range(K):
        q, il = divmod(i, hb)
        expect = np.zeros(K)
        expect[q * hb:(q + 1) * hb] = c[i] * Hs[:, il]
        assert np.allclose(xt[i], expect, rtol=0, atol=1e-14), f"T e_{i} wrong"


def pin_whiten_norm_and_diag(o, rp=None):
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 64))
    xt = o.whiten(x, np.ones(64), 16)
    assert np.allclose(np.linalg.norm(xt, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    c = rng.uniform(0.8, 1.2, 64)
    assert np.allclose(o.whiten(x, c, 1), x * c[None, :], rtol=1e-15, atol=0)


# ----------------------------------------------------------------- decoding

FIG2_CASES = [(2, 1), (4, 2), (5, 2), (8, 3)]   # (D, d)


def pin_codebook_bruteforce(o, rp=None):
    rng = np.random.default_rng(9)
    for D, d in FIG2_CASES:
        M = _dyadic(rng, (d, D))
        Mf = [[_frac(M[i, e]) for e in range(D)] for i in range(d)]
        N = 1 << D
        # Row n holds the sign pattern of the integer n (bit e set -> -1).
        signs = np.array([[[(-1 if (n >> e) & 1 else 1) for e in range(D)]]
                          for n in range(N)], dtype=np.int8)
        W = o.decode_weight(signs, M)
        assert W.shape == (N, d)
        for n in range(N):
            s = [(-1 if (n >> e) & 1 else 1) for e in range(D)]
            for i in range(d):
                exact = sum(Mf[i][e] * s[e] for e in range(D))
                assert _frac(W[n, i]) == exact, f"codeword {n} of ({D},{d}) wrong"
        # One block (K = d), T = I, unit row scale: y[n] = x . (M s_n), exact.
        x = _dyadic(rng, (1, d))
        y = o.linear(x, np.ones(d), 1, M, signs, np.ones(N))
        for n in range(N):
            s = [(-1 if (n >> e) & 1 else 1) for e in range(D)]
            exact = sum(_frac(x[0, i]) * sum(Mf[i][e] * s[e] for e in range(D))
                        for i in range(d))
            assert _frac(y[0, n]) == exact
        # Codebook enumeration and its moments over the full hypercube.
        cb = o.codebook(M)
        assert cb.shape == (N, d)
        assert np.array_equal(cb, W)
        mean = [sum(_frac(cb[n, i]) for n in range(N)) / N for i in range(d)]
        assert all(m == 0 for m in mean), "codebook mean must be exactly 0"
        for i in range(d):
            for k in range(d):
                second = sum(_frac(cb[n, i]) * _frac(cb[n, k]) for n in range(N)) / N
                mmt = sum(Mf[i][e] * Mf[k][e] for e in range(D))
                assert second == mmt, "codebook second moment must equal M M^T"


def pin_multiblock_bruteforce(o, rp=None):
    """K = 3d with independent patterns per block; exact with dyadic data."""
    rng = np.random.default_rng(10)
    for D, d in FIG2_CASES:
        Kb, N = 3, 16
        M = _dyadic(rng, (d, D))
        signs = _signs(rng, N, Kb, D)
        x = _dyadic(rng, (2, Kb * d))
        r = _dyadic(rng, (N,), denom=4, lim=6)
        y = o.linear(x, np.ones(Kb * d), 1, M, signs, r)
        for bt in range(2):
            for n in range(N):
                acc = Fraction(0)
                for b in range(Kb):
                    for i in range(d):
                        w = sum(_frac(M[i, e]) * int(signs[n, b, e]) for e in range(D))
                        acc += w * _frac(x[bt, b * d + i])
                assert _frac(y[bt, n]) == _frac(r[n]) * acc


def pin_identity_mapping(o, rp=None):
    """D = d and M = I: W equals the sign matrix; with T = I, unit scales and
    integer activations the operator is the integer product S @ x."""
    rng = np.random.default_rng(11)
    for d in [1, 3, 4]:
        N, Kb = 32, 5
        signs = _signs(rng, N, Kb, d)
        W = o.decode_weight(signs, np.eye(d))
        assert np.array_equal(W, signs.reshape(N, Kb * d).astype(np.float64))
        xi = rng.integers(-50, 51, size=(3, Kb * d))
        y = o.linear(xi.astype(np.float64), np.ones(Kb * d), 1, np.eye(d), signs, np.ones(N))
        ref = xi.astype(np.int64) @ signs.reshape(N, Kb * d).astype(np.int64).T
        assert np.array_equal(y, ref.astype(np.float64))


# ------------------------------------------------------- lifted route, scales

def pin_lifted_route(o, rp=None):
    """S (M^T T x) equals W (T x) (the rearrangement behind the fused
    operator), for K a multiple of d and not."""
    rng = np.random.default_rng(12)
    for (N, K, d, D, hb) in [(64, 512, 2, 5, 512), (48, 64, 10, 24, 32), (32, 96, 7, 9, 16)]:
        Kb = -(-K // d)
        M = rng.standard_normal((d, D)) / np.sqrt(D)
        signs = _signs(rng, N, Kb, D)
        c = rng.uniform(0.8, 1.2, K)
        r = rng.uniform(0.5, 1.5, N)
        x = rng.standard_normal((3, K))
        y = o.linear(x, c, hb, M, signs, r)
        z = o.lift(o.pad_blocks(o.whiten(x, c, hb), d), M)
        y2 = o.sign_matmul(signs.reshape(N, Kb * D), z, r)
        assert np.linalg.norm(y - y2) <= 1e-12 * np.linalg.norm(y)


def pin_lift_bruteforce(o, rp=None):
    rng = np.random.default_rng(13)
    d, D, Kb = 3, 8, 4
    M = _dyadic(rng, (d, D))
    xt = _dyadic(rng, (2, Kb * d))
    z = o.lift(xt, M)
    assert z.shape == (2, Kb * D)
    for bt in range(2):
        for b in range(Kb):
            for e in range(D):
                exact = sum(_frac(M[i, e]) * _frac(xt[bt, b * d + i]) for i in range(d))
                assert _frac(z[bt, b * D + e]) == exact


def pin_sign_matmul_integer(o, rp=None):
    rng = np.random.default_rng(14)
    S = _signs(rng, 48, 120)
    zi = rng.integers(-1000, 1001, size=(5, 120))
    y = o.sign_matmul(S, zi.astype(np.float64), np.ones(48))
    assert np.array_equal(y, (zi.astype(np.int64) @ S.astype(np.int64).T).astype(np.float64))
    r = rng.uniform(0.5, 1.5, 48)
    y2 = o.sign_matmul(S, zi.astype(np.float64), r)
    assert np.allclose(y2, y * r[None, :], rtol=1e-15, atol=0)


def pin_row_scale(o, rp=None):
    rng = np.random.default_rng(15)
    N, K, d, D, hb = 32, 64, 4, 9, 16
    M = rng.standard_normal((d, D))
    signs = _signs(rng, N, K // d, D)
    c = rng.uniform(0.8, 1.2, K)
    x = rng.standard_normal((2, K))
    r = rng.uniform(0.5, 1.5, N)
    y1 = o.linear(x, c, hb, M, signs, r)
    y2 = o.linear(x, c, hb, M, signs, 2 * r)
    assert np.allclose(y2, 2 * y1, rtol=1e-14, atol=0)
    onehot = np.zeros(N)
    onehot[5] = 1.0
    y3 = o.linear(x, c, hb, M, signs, onehot)
    assert np.all(y3[:, np.arange(N) != 5] == 0)
    assert np.allclose(y3[:, 5], y1[:, 5] / r[5], rtol=1e-13)


def pin_zero_pad(o, rp=None):
    """Virtual zero padding equals explicit zero channels."""
    rng = np.random.default_rng(16)
    N, K, d, D = 16, 12, 5, 7                   # K' = 15
    Kb = 3
    M = rng.standard_normal((d, D))
    signs = _signs(rng, N, Kb, D)
    c = rng.uniform(0.8, 1.2, K)
    r = rng.uniform(0.5, 1.5, N)
    x = rng.standard_normal((2, K))
    y = o.linear(x, c, 1, M, signs, r)
    xp = np.concatenate([x, np.zeros((2, 3))], axis=1)
    cp = np.concatenate([c, np.ones(3)])
    yp = o.linear(xp, cp, 1, M, signs, r)
    assert np.allclose(y, yp, rtol=1e-14, atol=1e-14)
    assert o.pad_blocks(x, d).shape == (2, 15)
    assert np.all(o.pad_blocks(x, d)[:, K:] == 0)
    assert np.array_equal(o.pad_blocks(x, d)[:, :K], x)


# ----------------------------------------------------------- storage, rates

def _golden_rates():
    rows = []
    for line in (GOLDEN / "rates.txt").read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if line:
            D, d, bits = line.split()[:3]
            rows.append((int(D), int(d), float(bits)))
    return rows


def pin_rates(o, rp=None):
    for D, d, bits in _golden_rates():
        for k in [1, 7, 410]:
            K = d * k
            assert round(o.bits_per_weight(K, d, D), 2) == bits
            assert o.packed_bits(64, K, d, D) == 64 * k * D
            assert round(o.packed_bits(64, K, d, D) / (64 * K), 2) == bits


def pin_memory_fit(o, rp=None):
    for line in (GOLDEN / "memory_fit.txt").read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        params_b, D, d, cap_gb, fits = line.split()[:5]
        params = int(float(params_b) * 1e9)
        # Count weights in d-blocks: ceil(params / d) blocks of D bits.
        nbytes = o.packed_bits(1, params, int(d), int(D)) / 8
        assert (nbytes <= float(cap_gb) * 1e9) == (fits == "yes"), line


def pin_storage_exact(o, rp):
    rng = np.random.default_rng(17)
    for (N, K, d, D) in [(16, 512, 2, 5), (32, 4096 // 8, 10, 24), (48, 100, 3, 8),
                         (16, 8, 1, 1), (64, 1500, 10, 24), (16, 3, 3, 8)]:
        Kb = -(-K // d)
        L = Kb * D
        if L % 8:
            continue
        S = _signs(rng, N, L)
        packed = rp.refpack(S)
        assert packed.size * 8 == o.packed_bits(N, K, d, D)
        assert np.array_equal(rp.refunpack(packed, N, L), S)


def pin_pack_layout_bijective(o, rp):
    for (N, L) in [(16, 8), (16, 512), (32, 1280), (16, 1544), (48, 9840 // 10 * 10 // 8 * 8)]:
        nn, jj = np.meshgrid(np.arange(N), np.arange(L), indexing="ij")
        idx = rp.bit_index(nn.ravel(), jj.ravel(), N, L)
        assert np.array_equal(np.sort(idx), np.arange(N * L)), "layout must be a bijection"


def pin_encode_bruteforce(o, rp):
    rng = np.random.default_rng(23)
    for (d, D) in [(1, 1), (1, 3), (2, 5), (3, 6), (4, 4), (2, 7)]:
        M = rng.standard_normal((d, D)) / np.sqrt(D)
        w = rng.standard_normal((9, d))
        signs, dist = o.encode_nn(w, M)
        assert signs.shape == (9, D) and dist.shape == (9,)
        for b in range(9):
            best, arg = None, None
            for s in itertools.product((1.0, -1.0), repeat=D):
                acc = 0.0
                for i in range(d):
                    v = w[b, i]
                    for e in range(D):
                        v -= M[i, e] * s[e]
                    acc += v * v
                if best is None or acc < best - 1e-12:
                    best, arg = acc, s
            assert np.array_equal(signs[b], np.array(arg)), (d, D, b)
            assert abs(dist[b] - best) <= 1e-12 * max(1.0, best)


def pin_encode_identity(o, rp):
    rng = np.random.default_rng(29)
    for d in (1, 3, 6):
        w = rng.standard_normal((20, d))
        w[0, 0] = 0.0                                  # a tie: both signs equally close
        signs, dist = o.encode_nn(w, np.eye(d))
        want = np.where(w >= 0, 1.0, -1.0)
        assert np.array_equal(signs, want)
        assert np.allclose(dist, ((np.abs(w) - 1.0) ** 2).sum(axis=1), rtol=0, atol=1e-12)


def pin_encode_symmetry(o, rp):
    rng = np.random.default_rng(31)
    M = rng.standard_normal((3, 8)) / np.sqrt(8)
    w = rng.standard_normal((40, 3))
    s, dist = o.encode_nn(w, M)
    s_neg, dist_neg = o.encode_nn(-w, M)
    assert np.array_equal(s_neg, -s)
    assert np.allclose(dist_neg, dist, rtol=1e-12, atol=0)
    s2, dist2 = o.encode_nn(2.0 * w, 2.0 * M)
    assert np.array_equal(s2, s)
    assert np.allclose(dist2, 4.0 * dist, rtol=1e-12, atol=0)


def _pinv_bruteforce(w, M):
    """The partial search written out candidate by candidate: for every sign
    vector of the last D - d columns (in pattern order), the first d signs
    from a linear solve (not a pseudo-inverse), the distance from a plain
    loop, ties to the lower full pattern index."""
    d, D = M.shape
    F = D - d
    best, arg, bidx = None, None, None
    for q in range(1 << F):
        sf = [(-1.0 if (q >> k) & 1 else 1.0) for k in range(F)]
        rhs = w - M[:, d:] @ np.array(sf) if F else w.copy()
        u = np.linalg.solve(M[:, :d], rhs)
        sa = [1.0 if v >= 0.0 else -1.0 for v in u]
        s = sa + sf
        acc = 0.0
        for i in range(d):
            v = w[i]
            for e in range(D):
                v -= M[i, e] * s[e]
            acc += v * v
        idx = sum(1 << e for e in range(D) if s[e] < 0)
        if best is None or acc < best or (acc == best and idx < bidx):
            best, arg, bidx = acc, s, idx
    return np.array(arg), best


def pin_encode_pinv_bruteforce(o, rp):
    rng = np.random.default_rng(47)
    for (d, D) in [(1, 1), (1, 4), (2, 5), (3, 6), (2, 2), (3, 8)]:
        M = rng.standard_normal((d, D)) / np.sqrt(D)
        w = rng.standard_normal((7, d))
        signs, dist = o.encode_pinv(w, M)
        assert signs.shape == (7, D) and dist.shape == (7,)
        for b in range(7):
            s, best = _pinv_bruteforce(w[b], M)
            assert np.array_equal(signs[b], s), (d, D, b)
            assert abs(dist[b] - best) <= 1e-12 * max(1.0, best)


def pin_encode_pinv_diagonal_exact(o, rp):
    """M_a diagonal: the per-coordinate signs of pinv(M_a) (w - M_f s_f) are
    the exact minimiser over s_a, so the partial search is the exhaustive one."""
    rng = np.random.default_rng(53)
    for (d, D) in [(1, 6), (2, 7), (3, 9), (4, 12), (5, 5)]:
        Ma = np.diag(rng.uniform(0.3, 1.5, d) * rng.choice([-1.0, 1.0], d))
        M = np.hstack([Ma, rng.standard_normal((d, D - d)) / np.sqrt(D)])
        w = rng.standard_normal((25, d))
        s1, d1 = o.encode_pinv(w, M)
        s2, d2 = o.encode_nn(w, M)
        assert np.array_equal(s1, s2), (d, D)
        assert np.allclose(d1, d2, rtol=1e-12, atol=1e-14)


def pin_encode_pinv_subset(o, rp):
    """Gaussian M: never closer than the exhaustive search, and the distance
    returned is that of the signs returned."""
    rng = np.random.default_rng(59)
    for (d, D) in [(2, 6), (4, 12), (3, 11)]:
        M = rng.standard_normal((d, D)) / np.sqrt(D)
        w = rng.standard_normal((40, d))
        s1, d1 = o.encode_pinv(w, M)
        _, d2 = o.encode_nn(w, M)
        assert np.all(d1 >= d2 - 1e-12)
        r = w - s1 @ M.T
        assert np.allclose(d1, (r * r).sum(axis=1), rtol=1e-12, atol=1e-14)
        assert np.all(np.abs(s1) == 1.0)


def pin_encode_pinv_square(o, rp):
    """D = d: a single candidate, the signs of the solution of M s = w (+1 at
    an exact zero)."""
    rng = np.random.default_rng(61)
    for d in (1, 3, 6):
        M = np.diag(rng.uniform(0.5, 2.0, d))
        w = rng.standard_normal((12, d))
        w[rng.random((12, d)) < 0.25] = 0.0
        s, dist = o.encode_pinv(w, M)
        assert np.array_equal(s, np.where(w >= 0.0, 1.0, -1.0))
        G = rng.standard_normal((d, d))
        s, _ = o.encode_pinv(w, G)
        assert np.array_equal(s, np.where(np.linalg.solve(G, w.T).T >= 0.0, 1.0, -1.0))


def _eq1_loss(o, M, w):
    """mean_b min_s ||w_b - M s|| evaluated from scratch (codebook distances)."""
    cb = o.codebook(M)
    dist = ((w[:, None, :] - cb[None, :, :]) ** 2).sum(axis=2)
    return float(np.sqrt(dist.min(axis=1)).mean()), dist.argmin(axis=1)


def pin_train_gradient_fd(o, rp):
    rng = np.random.default_rng(37)
    d, D = 2, 5
    M = rng.standard_normal((d, D)) / np.sqrt(D)
    w = rng.standard_normal((64, d))
    lr = 1e-3
    M_new, loss = o.train_m_step(M, w, lr)
    l0, arg0 = _eq1_loss(o, M, w)
    assert abs(loss - l0) <= 1e-12
    grad = (M - M_new) / lr
    h = 1e-6
    for i in range(d):
        for e in range(D):
            E = np.zeros_like(M)
            E[i, e] = h
            lp, argp = _eq1_loss(o, M + E, w)
            lm, argm = _eq1_loss(o, M - E, w)
            assert np.array_equal(argp, arg0) and np.array_equal(argm, arg0)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i, e]) <= 1e-6 * max(1.0, abs(fd)), (i, e, fd, grad[i, e])


def pin_train_descends(o, rp):
    rng = np.random.default_rng(41)
    G = rng.standard_normal((8, 8))
    M = o.orthonormal_rows(G, 3)
    w = rng.standard_normal((2000, 3))
    M1, l0 = o.train_m_step(M, w, 0.02)
    l1, _ = _eq1_loss(o, M1, w)
    assert l1 < l0, (l0, l1)
    assert abs(l0 - _eq1_loss(o, M, w)[0]) <= 1e-12


def pin_orthonormal_rows(o, rp):
    rng = np.random.default_rng(43)
    for (d, D) in [(3, 8), (10, 24), (4, 4)]:
        G = rng.standard_normal((D, D))
        M = o.orthonormal_rows(G, d)
        assert M.shape == (d, D)
        assert np.allclose(M @ M.T, np.eye(d), rtol=0, atol=1e-12)
        # the rows span the same space as the first d columns of G (Gram-Schmidt)
        proj = M.T @ M
        assert np.allclose(proj @ G[:, :d], G[:, :d], rtol=0, atol=1e-10)


ALL_PINS = [
    pin_hadamard_library, pin_hadamard_structure, pin_whiten_unit_vectors,
    pin_whiten_norm_and_diag, pin_codebook_bruteforce, pin_multiblock_bruteforce,
    pin_identity_mapping, pin_lifted_route, pin_lift_bruteforce,
    pin_sign_matmul_integer, pin_row_scale, pin_zero_pad, pin_rates,
    pin_memory_fit, pin_storage_exact, pin_pack_layout_bijective,
    pin_encode_bruteforce, pin_encode_identity, pin_encode_symmetry,
    pin_encode_pinv_bruteforce, pin_encode_pinv_diagonal_exact, pin_encode_pinv_subset,
    pin_encode_pinv_square,
    pin_train_gradient_fd, pin_train_descends, pin_orthonormal_rows,
]
