"""Plant plausible mistakes in copies of the CPU oracle and require that at
least one pin catches each of them (no GPU).

Every mutant is a fresh copy of ``oracle/liftquant_ref.py`` (or
``oracle/refpack.py``) with one function replaced; the real oracle is never
modified.
"""
import importlib.util
import itertools
from pathlib import Path

import numpy as np
import pytest

from tests import oracle_pins

ORACLE_DIR = Path(__file__).resolve().parent.parent / "oracle"
_counter = itertools.count()


def _fresh(name):
    spec = importlib.util.spec_from_file_location(
        f"_mutant_{name}_{next(_counter)}", ORACLE_DIR / f"{name}.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _mutants():
    out = []

    def m(desc):
        def deco(fn):
            out.append((desc, fn))
            return fn
        return deco

    @m("Hadamard without 1/sqrt(hb)")
    def _(o, rp):
        orig = o.hadamard
        o.hadamard = lambda hb: orig(hb) * np.sqrt(hb)

    @m("Hadamard sign from popcount(i | j)")
    def _(o, rp):
        def h(hb):
            i = np.arange(hb)
            par = o._popcount(i[:, None] | i[None, :]) % 2
            return np.where(par == 0, 1.0, -1.0) / np.sqrt(hb)
        o.hadamard = h

    @m("channel scale applied after mixing")
    def _(o, rp):
        def whiten(x, c, hb):
            x = np.asarray(x, float)
            c = np.asarray(c, float)
            xt = np.empty_like(x)
            for q in range(x.shape[1] // hb):
                sl = slice(q * hb, (q + 1) * hb)
                xt[:, sl] = (x[:, sl] @ o.hadamard(hb).T) * c[sl]
            return xt
        o.whiten = whiten

    @m("channel scales of the wrong block")
    def _(o, rp):
        def whiten(x, c, hb):
            x = np.asarray(x, float)
            c = np.roll(np.asarray(c, float), hb)
            xt = np.empty_like(x)
            for q in range(x.shape[1] // hb):
                sl = slice(q * hb, (q + 1) * hb)
                xt[:, sl] = x[:, sl] @ o.whitening_block(c[sl]).T
            return xt
        o.whiten = whiten

    @m("mixing matrix transposed with scale (diag(c) H)")
    def _(o, rp):
        o.whitening_block = lambda cb: np.diag(np.asarray(cb, float)) @ o.hadamard(len(cb))

    @m("decoded block uses the sign vector negated")
    def _(o, rp):
        orig = o.decode_weight
        o.decode_weight = lambda s, M: orig(-np.asarray(s), M)

    @m("decoded block drops the last sign")
    def _(o, rp):
        def dw(signs, M):
            s = np.array(signs, dtype=np.int64)
            s[:, :, -1] = 0
            return o.__dict__["_orig_dw"](s, M)
        o._orig_dw = o.decode_weight
        o.decode_weight = dw

    @m("decoded blocks in reverse order")
    def _(o, rp):
        orig = o.decode_weight
        o.decode_weight = lambda s, M: orig(np.asarray(s)[:, ::-1, :], M)

    @m("mapping matrix read with swapped index (square M)")
    def _(o, rp):
        orig = o.decode_weight

        def dw(s, M):
            M = np.asarray(M, float)
            return orig(s, M.T if M.shape[0] == M.shape[1] else M[:, ::-1])
        o.decode_weight = dw

    @m("row scale ignored")
    def _(o, rp):
        orig = o.linear
        o.linear = lambda x, c, hb, M, s, r: orig(x, c, hb, M, s, np.ones_like(np.asarray(r, float)))

    @m("zero padding at the front")
    def _(o, rp):
        def pad(xt, d):
            xt = np.asarray(xt, float)
            B, K = xt.shape
            Kp = -(-K // d) * d
            out = np.zeros((B, Kp))
            out[:, Kp - K:] = xt
            return out
        o.pad_blocks = pad

    @m("lift uses M^T x with the block stride of D")
    def _(o, rp):
        def lift(xt, M):
            xt = np.asarray(xt, float)
            M = np.asarray(M, float)
            d, D = M.shape
            Kb = xt.shape[1] // d
            z = np.zeros((xt.shape[0], Kb * D))
            for b in range(Kb):
                lo = min(b * D, xt.shape[1] - d)
                z[:, b * D:(b + 1) * D] = xt[:, lo:lo + d] @ M
            return z
        o.lift = lift

    @m("lift with M columns reversed")
    def _(o, rp):
        orig = o.lift
        o.lift = lambda xt, M: orig(xt, np.asarray(M, float)[:, ::-1])

    @m("sign matmul without row scale")
    def _(o, rp):
        orig = o.sign_matmul
        o.sign_matmul = lambda S, z, r: orig(S, z, np.ones(np.asarray(r).shape))

    @m("storage uses floor(K/d)")
    def _(o, rp):
        o.packed_bits = lambda N, K, d, D: N * (K // d) * D

    @m("bits per weight ignores the block length")
    def _(o, rp):
        o.bits_per_weight = lambda K, d, D: float(D)

    @m("codebook pattern off by one bit")
    def _(o, rp):
        o.sign_pattern = lambda i, D: np.array(
            [-1.0 if (i >> ((e + 1) % D)) & 1 else 1.0 for e in range(D)])

    @m("packed tail rows interleaved like full tiles")
    def _(o, rp):
        orig = rp.bit_index

        def bi(n, j, N, L):
            idx = orig(n, j, N, L)
            return np.where(np.asarray(j) >= (L // 512) * 512, idx // 2, idx)
        rp.bit_index = bi

    @m("packed slot ignores the column group")
    def _(o, rp):
        orig = rp.bit_index

        def bi(n, j, N, L):
            j = np.asarray(j)
            return orig(n, np.where(j % 128 >= 32, j - 32, j), N, L)
        rp.bit_index = bi

    @m("encoder picks the farthest codeword")
    def _(o, rp):
        def enc(w, M):
            M = np.asarray(M, float)
            d, D = M.shape
            w = np.asarray(w, float).reshape(-1, d)
            cb = o.codebook(M)
            dist = ((w[:, None, :] - cb[None, :, :]) ** 2).sum(axis=2)
            i = dist.argmax(axis=1)
            return np.stack([o.sign_pattern(int(k), D) for k in i]), dist[np.arange(len(i)), i]
        o.encode_nn = enc

    @m("encoder returns the complement of the chosen signs")
    def _(o, rp):
        orig = o.encode_nn

        def enc(w, M):
            s, dist = orig(w, M)
            return -s, dist
        o.encode_nn = enc

    @m("encoder breaks ties toward the highest index")
    def _(o, rp):
        def enc(w, M):
            M = np.asarray(M, float)
            d, D = M.shape
            w = np.asarray(w, float).reshape(-1, d)
            cb = o.codebook(M)
            dist = ((w[:, None, :] - cb[None, :, :]) ** 2).sum(axis=2)
            i = (dist.shape[1] - 1) - dist[:, ::-1].argmin(axis=1)
            return np.stack([o.sign_pattern(int(k), D) for k in i]), dist[np.arange(len(i)), i]
        o.encode_nn = enc

    @m("partial search solves for the last d columns")
    def _(o, rp):
        orig = o.encode_pinv

        def enc(w, M):
            M = np.asarray(M, float)
            d, D = M.shape
            perm = list(range(D - d, D)) + list(range(D - d))
            s, dist = orig(w, M[:, perm])
            out = np.zeros_like(s)
            out[:, perm] = s
            return out, dist
        o.encode_pinv = enc

    @m("partial search rounds the solved coordinates with sgn(0) = -1")
    def _(o, rp):
        orig = o.encode_pinv

        def enc(w, M):
            w = np.asarray(w, float)
            M = np.asarray(M, float)
            d = M.shape[0]
            return orig(np.where(w.reshape(-1, d) == 0.0, -1e-300, w), M)
        o.encode_pinv = enc

    @m("partial search keeps the farthest candidate")
    def _(o, rp):
        def enc(w, M):
            M = np.asarray(M, float)
            d, D = M.shape
            F = D - d
            w = np.asarray(w, float).reshape(-1, d)
            A = np.linalg.pinv(M[:, :d])
            q = np.arange(1 << F)
            Sf = np.where((q[:, None] >> np.arange(F)[None, :]) & 1, -1.0, 1.0)
            out, dd = np.zeros((len(w), D)), np.zeros(len(w))
            for b in range(len(w)):
                U = (A @ (w[b][:, None] - M[:, d:] @ Sf.T)).T
                Sa = np.where(U >= 0, 1.0, -1.0)
                R = w[b] - Sa @ M[:, :d].T - Sf @ M[:, d:].T
                dist = (R * R).sum(axis=1)
                k = int(dist.argmax())
                out[b, :d], out[b, d:], dd[b] = Sa[k], Sf[k], dist[k]
            return out, dd
        o.encode_pinv = enc

    @m("partial search leaves the enumerated columns out of the solve")
    def _(o, rp):
        def enc(w, M):
            M = np.asarray(M, float)
            d, D = M.shape
            F = D - d
            w = np.asarray(w, float).reshape(-1, d)
            A = np.linalg.pinv(M[:, :d])
            q = np.arange(1 << F)
            Sf = np.where((q[:, None] >> np.arange(F)[None, :]) & 1, -1.0, 1.0)
            out, dd = np.zeros((len(w), D)), np.zeros(len(w))
            for b in range(len(w)):
                sa = np.where(A @ w[b] >= 0, 1.0, -1.0)
                R = w[b] - sa @ M[:, :d].T - Sf @ M[:, d:].T
                dist = (R * R).sum(axis=1)
                k = int(dist.argmin())
                out[b, :d], out[b, d:], dd[b] = sa, Sf[k], dist[k]
            return out, dd
        o.encode_pinv = enc

    @m("training step ascends")
    def _(o, rp):
        orig = o.train_m_step

        def step(M, w, lr):
            return orig(M, w, -lr)
        o.train_m_step = step

    @m("training step uses the squared norm")
    def _(o, rp):
        def step(M, w, lr):
            M = np.asarray(M, float)
            d, D = M.shape
            w = np.asarray(w, float).reshape(-1, d)
            s, _ = o.encode_nn(w, M)
            r = w - s @ M.T
            loss = float(np.sqrt((r * r).sum(axis=1)).mean())
            grad = -2.0 * (r.T @ s) / w.shape[0]
            return M - lr * grad, loss
        o.train_m_step = step

    @m("initial M with orthonormal columns of a tall draw")
    def _(o, rp):
        def orth(G, d):
            q, _ = np.linalg.qr(np.asarray(G, float)[:, :d])
            return q.T[:, :G.shape[0]] * 1.5
        o.orthonormal_rows = orth

    return out


MUTANTS = _mutants()


@pytest.mark.parametrize("desc,mutate", MUTANTS, ids=[d for d, _ in MUTANTS])
def test_mutant_is_caught(desc, mutate):
    o = _fresh("liftquant_ref")
    rp = _fresh("refpack")
    mutate(o, rp)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o, rp)
        except Exception as exc:  # any failure (assertion or crash) counts
            caught.append(f"{pin.__name__}: {type(exc).__name__}")
    assert caught, f"no pin catches the planted mistake: {desc}"
