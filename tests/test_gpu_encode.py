"""Parity of the nearest-neighbour encoder (lq_encode) and of the training
step of M (lq_train_m_step) with the CPU oracle.

* Encoding: synthetic N(0, I_d) blocks ([paper] §3.1 trains and measures M
  on them), M with orthonormal rows or Gaussian entries; every (d, D) on the
  pages' rates that the oracle's exhaustive search finishes in seconds
  (D <= 20), both search layouts (a lane per block for D <= 10, a wavefront
  per block beyond), a ragged block count. The chosen sign vectors must be
  the oracle's (random data has no ties) and the squared distances agree to
  float rounding. D = 24 (the 2.4-bit rate) at full search: properties that
  hold at any size (no single sign flip gets closer; odd symmetry), and the
  oracle on a few blocks.
* Ties: M = I with exact zeros in w: the lowest index (s = +1) must win.
* End to end: a weight matrix encoded, packed and run through lq_linear
  matches the oracle's operator with the encoded signs.
* Training: one step of M against the oracle's step (fp64 on both sides,
  M stored as fp32), the loss, several steps decreasing the loss, and
  determinism.
* The 2^(D-d) pseudo-inverse-initialised search (lq_encode_pinv) against the
  oracle's ``encode_pinv``: both layouts (a lane per block for D - d <= 10, a
  wavefront beyond), LQ-24/10 and LQ-32/16 (2^16 candidates per block),
  D = d; the chosen sign vectors must be the oracle's and the distances agree
  to float rounding. With a diagonal M_a it is the exhaustive search, so it
  must equal lq_encode. A singular M_a and a short workspace are errors.
"""
import numpy as np
import pytest
import torch

from oracle import liftquant_ref as ref
from tests.gpu_util import DeviceLayer, dev, host, note, rel_l2
from workloads import make_layer_small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lq():
    import bit_matmul_amd
    assert torch.cuda.is_available()
    return bit_matmul_amd


def _gpu_encode(lq, w, M):
    n, d = w.shape
    D = M.shape[1]
    wd = dev(w.astype(np.float32))
    Md = dev(M.astype(np.float32))
    signs = torch.zeros((n, D), dtype=torch.int8, device="cuda")
    dist = torch.zeros(n, dtype=torch.float32, device="cuda")
    note(f"lq_encode n={n} d={d} D={D}")
    lq.lq_encode(wd, n, d, D, Md, signs, dist)
    torch.cuda.synchronize()
    return signs.cpu().numpy().astype(np.float64), dist.cpu().numpy().astype(np.float64)


def _dist(w, M, s):
    r = w - s @ M.T
    return (r * r).sum(axis=1)


CASES = [
    # (d, D, n)
    (1, 1, 37), (2, 5, 300), (3, 8, 513), (4, 4, 100), (2, 10, 257),
    (10, 12, 70), (2, 11, 65), (3, 14, 33), (10, 16, 9), (16, 16, 5), (10, 20, 3),
]


@pytest.mark.parametrize("d,D,n", CASES, ids=[f"d{c[0]}-D{c[1]}" for c in CASES])
@pytest.mark.parametrize("init", ["orthonormal", "gaussian"])
def test_encode_matches_oracle(lq, d, D, n, init):
    rng = np.random.default_rng(1000 * d + D)
    if init == "orthonormal":
        M = ref.orthonormal_rows(rng.standard_normal((D, D)), d)
    else:
        M = rng.standard_normal((d, D)) / np.sqrt(D)
    M = M.astype(np.float32).astype(np.float64)     # the values the GPU sees
    w = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    s_gpu, d_gpu = _gpu_encode(lq, w, M)
    s_ref, d_ref = ref.encode_nn(w, M)
    assert np.array_equal(s_gpu, s_ref)
    assert np.allclose(d_gpu, d_ref, rtol=1e-6, atol=1e-7)


def test_encode_ties_lowest_index(lq):
    rng = np.random.default_rng(5)
    for d in (1, 4, 9):
        w = rng.standard_normal((64, d))
        w[rng.random((64, d)) < 0.3] = 0.0              # exact ties on those coordinates
        s_gpu, d_gpu = _gpu_encode(lq, w, np.eye(d))
        s_ref, _ = ref.encode_nn(w, np.eye(d))
        assert np.array_equal(s_gpu, s_ref)
        assert np.array_equal(s_gpu, np.where(w >= 0, 1.0, -1.0))


def test_encode_rate_24_properties(lq):
    """d = 10, D = 24 (2.4 bits): 2^24 sign vectors per block."""
    rng = np.random.default_rng(24)
    M = ref.orthonormal_rows(rng.standard_normal((24, 24)), 10).astype(np.float32).astype(np.float64)
    w = rng.standard_normal((64, 10)).astype(np.float32).astype(np.float64)
    s, dist = _gpu_encode(lq, w, M)
    base = _dist(w, M, s)
    assert np.allclose(dist, base, rtol=1e-6, atol=1e-7)
    for e in range(24):                                 # no single flip gets closer
        t = s.copy()
        t[:, e] = -t[:, e]
        assert np.all(_dist(w, M, t) >= base - 1e-12)
    s_neg, _ = _gpu_encode(lq, -w, M)
    assert np.array_equal(s_neg, -s)
    s_ref, d_ref = ref.encode_nn(w[:2], M)              # the oracle on two blocks
    assert np.array_equal(s[:2], s_ref)
    assert np.allclose(dist[:2], d_ref, rtol=1e-6)


def test_encode_pack_linear_end_to_end(lq):
    """A weight matrix in the lifted frame encoded, packed and applied."""
    N, K, d, D, hb = 64, 1024, 3, 8, 512
    inp = make_layer_small(N, K, d, D, hb, seed=88, B_max=4, xdtype="f32")
    Kb = -(-K // d)
    rng = np.random.default_rng(88)
    Wblk = rng.standard_normal((N * Kb, d)).astype(np.float32)
    signs = torch.zeros((N * Kb, D), dtype=torch.int8, device="cuda")
    lq.lq_encode(dev(Wblk), N * Kb, d, D, dev(inp.M.astype(np.float32)), signs)
    torch.cuda.synchronize()
    s_ref, _ = ref.encode_nn(Wblk.astype(np.float64), inp.M.astype(np.float64))
    assert np.array_equal(signs.cpu().numpy().astype(np.float64), s_ref)
    # the layer with these signs, through lq_pack_signs and lq_linear
    inp._signs = s_ref.reshape(N, Kb, D).astype(np.int8)
    inp.signs = lambda: inp._signs
    layer = DeviceLayer(inp, lq)
    x = inp.x(3)
    y = layer.linear(lq, dev(x), 3, torch.float32)
    want = ref.linear(x, inp.c, hb, inp.M, inp._signs, inp.row_scale)
    assert rel_l2(host(y), want) < 1e-4


def _gpu_train(lq, M, w, lr, steps=1):
    n, d = w.shape
    D = M.shape[1]
    Md = dev(M.astype(np.float32))
    wd = dev(w.astype(np.float32))
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = torch.zeros(lq.lq_train_m_step_workspace_size(n, d, D), dtype=torch.uint8, device="cuda")
    losses = []
    for _ in range(steps):
        note(f"lq_train_m_step n={n} d={d} D={D}")
        lq.lq_train_m_step(Md, wd, n, d, D, lr, loss, ws)
        losses.append(float(loss.cpu()))
    torch.cuda.synchronize()
    return Md.cpu().numpy().astype(np.float64), losses


@pytest.mark.parametrize("d,D,n", [(2, 5, 4096), (3, 8, 1000), (4, 8, 777), (2, 12, 300)])
def test_train_step_matches_oracle(lq, d, D, n):
    rng = np.random.default_rng(7 * d + D)
    M = ref.orthonormal_rows(rng.standard_normal((D, D)), d).astype(np.float32).astype(np.float64)
    w = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    lr = 0.05
    M_gpu, (loss_gpu,) = _gpu_train(lq, M, w, lr)
    M_ref, loss_ref = ref.train_m_step(M, w, lr)
    assert abs(loss_gpu - loss_ref) <= 1e-6 * loss_ref
    assert np.allclose(M_gpu, M_ref, rtol=0, atol=2e-7 * max(1.0, np.abs(M_ref).max()))


def test_train_descends_and_is_deterministic(lq):
    rng = np.random.default_rng(99)
    d, D = 3, 8
    M0 = ref.orthonormal_rows(rng.standard_normal((D, D)), d)
    w = rng.standard_normal((8192, d))
    M1, losses = _gpu_train(lq, M0, w, 0.05, steps=20)
    assert losses[-1] < losses[0]
    M2, losses2 = _gpu_train(lq, M0, w, 0.05, steps=20)
    assert np.array_equal(M1, M2) and losses == losses2
    # the oracle's 20 steps land on the same M (fp32 storage between steps)
    Mr = M0.astype(np.float32).astype(np.float64)
    wr = w.astype(np.float32).astype(np.float64)
    for _ in range(20):
        Mr, _ = ref.train_m_step(Mr, wr, 0.05)
        Mr = Mr.astype(np.float32).astype(np.float64)
    assert np.allclose(M1, Mr, rtol=0, atol=1e-5)


def _gpu_encode_pinv(lq, w, M):
    n, d = w.shape
    D = M.shape[1]
    wd = dev(w.astype(np.float32))
    Md = dev(M.astype(np.float32))
    signs = torch.zeros((n, D), dtype=torch.int8, device="cuda")
    dist = torch.zeros(n, dtype=torch.float32, device="cuda")
    ws = torch.zeros(lq.lq_encode_pinv_workspace_size(d, D), dtype=torch.uint8, device="cuda")
    note(f"lq_encode_pinv n={n} d={d} D={D}")
    lq.lq_encode_pinv(wd, n, d, D, Md, signs, dist, ws)
    torch.cuda.synchronize()
    return signs.cpu().numpy().astype(np.float64), dist.cpu().numpy().astype(np.float64)


PINV_CASES = [
    # (d, D, n): D - d <= 10 a lane per block, beyond a wavefront per block
    (1, 1, 20), (1, 6, 37), (2, 5, 300), (3, 8, 129), (4, 4, 50), (2, 12, 65),
    (2, 13, 33), (12, 16, 17), (5, 20, 5), (10, 24, 9), (16, 32, 4),
]


@pytest.mark.parametrize("d,D,n", PINV_CASES, ids=[f"d{c[0]}-D{c[1]}" for c in PINV_CASES])
@pytest.mark.parametrize("init", ["orthonormal", "gaussian"])
def test_encode_pinv_matches_oracle(lq, d, D, n, init):
    rng = np.random.default_rng(7000 + 100 * d + D)
    if init == "orthonormal":
        M = ref.orthonormal_rows(rng.standard_normal((D, D)), d)
    else:
        M = rng.standard_normal((d, D)) / np.sqrt(D)
    M = M.astype(np.float32).astype(np.float64)
    w = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    s_gpu, d_gpu = _gpu_encode_pinv(lq, w, M)
    s_ref, d_ref = ref.encode_pinv(w, M)
    assert np.array_equal(s_gpu, s_ref)
    assert np.allclose(d_gpu, d_ref, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("d,D", [(3, 12), (10, 20), (4, 16), (1, 9)])
def test_encode_pinv_diagonal_is_exhaustive(lq, d, D):
    rng = np.random.default_rng(8000 + 100 * d + D)
    Ma = np.diag(rng.uniform(0.3, 1.5, d) * rng.choice([-1.0, 1.0], d))
    M = np.hstack([Ma, rng.standard_normal((d, D - d)) / np.sqrt(D)]).astype(np.float32).astype(np.float64)
    w = rng.standard_normal((33, d)).astype(np.float32).astype(np.float64)
    s_p, d_p = _gpu_encode_pinv(lq, w, M)
    s_e, d_e = _gpu_encode(lq, w, M)
    assert np.array_equal(s_p, s_e)
    assert np.allclose(d_p, d_e, rtol=1e-6, atol=1e-7)


def test_encode_pinv_errors(lq):
    d, D = 3, 8
    M = np.ones((d, D))                                  # M_a of rank 1
    w = np.zeros((4, d))
    with pytest.raises(lq.LQError) as e:
        _gpu_encode_pinv(lq, w, M)
    assert e.value.status == lq._lib.LQ_ERR_INVALID_ARG
    wd = dev(w.astype(np.float32))
    Md = dev(np.eye(d, D).astype(np.float32))
    signs = torch.zeros((4, D), dtype=torch.int8, device="cuda")
    short = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(lq.LQError) as e:
        lq.lq_encode_pinv(wd, 4, d, D, Md, signs, None, short)
    assert e.value.status == lq._lib.LQ_ERR_WORKSPACE
