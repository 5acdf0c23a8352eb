"""Parity of each kernel entry point with the CPU oracle (MI355X only).

Sizes span several 512-column packed tiles plus ragged tails; every input is
seeded. Bars: packing is bit-exact; fp32 results are within rel-L2 1e-4 of
the fp64 oracle (observed ~1e-7); bf16 results within 1e-2.
"""
import numpy as np
import pytest
import torch

from oracle import liftquant_ref as ref
from oracle import refpack as rp
from tests.gpu_util import DEV, dev, host, note, rel_l2, sign_gemm
from workloads import WORKLOADS, bf16_round, make_layer, make_layer_small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lq():
    import bit_matmul_amd
    assert torch.cuda.is_available()
    return bit_matmul_amd


def _signs(seed, N, L):
    rng = np.random.default_rng(seed)
    return np.where(rng.random((N, L)) < 0.5, -1, 1).astype(np.int8)


# ------------------------------------------------------------------ packing

PACK_SHAPES = [(16, 8), (16, 512), (32, 1280), (16, 1544), (48, 9840), (64, 21848), (16, 4104)]


@pytest.mark.parametrize("N,L", PACK_SHAPES)
def test_pack_bit_exact(lq, N, L):
    S = _signs(N * 7 + L, N, L)
    packed = torch.empty(N * L // 8, dtype=torch.uint8, device=DEV)
    note(f"pack N={N} L={L}")
    # d = 1, D = 1 gives K = L lifted columns directly
    lq.lq_pack_signs(dev(S), N, L, 1, 1, packed)
    got = host(packed)
    assert np.array_equal(got, rp.refpack(S))
    back = torch.empty((N, L), dtype=torch.int8, device=DEV)
    lq.lq_unpack_signs(packed, N, L, 1, 1, back)
    assert np.array_equal(host(back), S)


def test_pack_any_negative_value_is_minus_one(lq):
    N, L = 16, 520
    rng = np.random.default_rng(3)
    vals = rng.integers(-128, 128, size=(N, L)).astype(np.int8)
    vals[vals == 0] = 1
    packed = torch.empty(N * L // 8, dtype=torch.uint8, device=DEV)
    lq.lq_pack_signs(dev(vals), N, L, 1, 1, packed)
    assert np.array_equal(host(packed), rp.refpack(np.where(vals < 0, -1, 1)))


@pytest.mark.parametrize("wl,li", [(w, i) for w in WORKLOADS for i in range(len(WORKLOADS[w].layers))])
def test_pack_full_size_sampled_panels(lq, wl, li):
    spec = WORKLOADS[wl].layers[li]
    inp = make_layer(spec, WORKLOADS[wl], B_max=1)
    N, L = spec.N, spec.L
    S = inp.signs().reshape(N, L)
    packed = torch.empty(N * L // 8, dtype=torch.uint8, device=DEV)
    note(f"pack full {wl}/{spec.name} N={N} L={L}")
    lq.lq_pack_signs(dev(S), N, spec.K, spec.d, spec.D, packed)
    torch.cuda.synchronize()
    got = host(packed)
    panels = sorted({0, N // 16 - 1, (N // 16) // 2, (N // 16) // 3})
    for p in panels:
        want = rp.refpack_panel(S[16 * p:16 * p + 16], L)
        assert np.array_equal(got[p * 2 * L:(p + 1) * 2 * L], want), f"panel {p}"
    back = torch.empty((N, L), dtype=torch.int8, device=DEV)
    lq.lq_unpack_signs(packed, N, spec.K, spec.d, spec.D, back)
    assert torch.equal(back, dev(S))


# ---------------------------------------------------------------- whitening

@pytest.mark.parametrize("hb", [1, 2, 4, 8, 16, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("xdtype", [torch.float32, torch.bfloat16])
def test_hadamard_scale(lq, hb, xdtype):
    rng = np.random.default_rng(hb)
    B, K = 3, max(hb, 8) * 5
    x = rng.standard_normal((B, K)).astype(np.float32)
    if xdtype == torch.bfloat16:
        x = bf16_round(x)
    c = rng.uniform(0.8, 1.2, K).astype(np.float32)
    xt = torch.empty((B, K), dtype=torch.float32, device=DEV)
    note(f"hadamard hb={hb} B={B} K={K} {xdtype}")
    lq.lq_hadamard_scale(dev(x, xdtype), B, K, hb, dev(c), xt)
    torch.cuda.synchronize()
    assert rel_l2(host(xt), ref.whiten(x, c, hb)) < 2e-6


@pytest.mark.parametrize("K,hb,B", [(4096, 1024, 1), (14336, 1024, 2), (512, 512, 1), (27648, 1024, 1)])
def test_hadamard_scale_model_shapes(lq, K, hb, B):
    rng = np.random.default_rng(K)
    x = bf16_round(rng.standard_normal((B, K)).astype(np.float32))
    c = rng.uniform(0.8, 1.2, K).astype(np.float32)
    xt = torch.empty((B, K), dtype=torch.float32, device=DEV)
    lq.lq_hadamard_scale(dev(x, torch.bfloat16), B, K, hb, dev(c), xt)
    torch.cuda.synchronize()
    assert rel_l2(host(xt), ref.whiten(x, c, hb)) < 2e-6


# --------------------------------------------------------------------- lift

@pytest.mark.parametrize("d,D,K", [(10, 24, 4096), (10, 24, 1037), (2, 5, 512), (3, 8, 8192),
                                   (1, 1, 64), (16, 32, 96), (64, 64, 200), (7, 9, 50)])
@pytest.mark.parametrize("zdtype", [torch.float32, torch.bfloat16])
def test_lift(lq, d, D, K, zdtype):
    rng = np.random.default_rng(d * 100 + D + K)
    B = 3
    Kb = -(-K // d)
    L = Kb * D
    xt = rng.standard_normal((B, K)).astype(np.float32)
    M = (rng.standard_normal((d, D)) / np.sqrt(D)).astype(np.float32)
    z = torch.empty((B, L), dtype=zdtype, device=DEV)
    note(f"lift d={d} D={D} K={K} {zdtype}")
    lq.lq_lift_activations(dev(xt), B, K, d, D, dev(M), z)
    torch.cuda.synchronize()
    want = ref.lift(ref.pad_blocks(xt, d), M)
    got = host(z)
    if zdtype == torch.float32:
        assert rel_l2(got, want) < 1e-6
    else:
        # bf16 output: every value within one bf16 rounding of the exact one
        assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-30)


# -------------------------------------------------------------- sign product

ALGOS = {"valu": 1, "mfma_small": 2, "mfma_large": 3}
SIGN_CASES = [
    # (N, L, B)
    (64, 1280, 1), (32, 9840, 1), (48, 2048, 2), (16, 1544, 3), (64, 4104, 4),
    (32, 1000, 5), (16, 3000, 8), (64, 1536, 13), (32, 2568, 16),
]


def _sign_inputs(N, L, B, seed, zdtype):
    rng = np.random.default_rng(seed)
    S = _signs(seed, N, L)
    z = rng.standard_normal((B, L)).astype(np.float32)
    if zdtype == torch.bfloat16:
        z = bf16_round(z)
    r = rng.uniform(0.5, 1.5, N).astype(np.float32)
    return S, z, r


def sign_tol(algo, zdtype, B):
    """Expected accuracy of each algorithm against the fp64 product of the
    same z values. VALU: fp32 accumulation only. Large MFMA: bf16 z is exact
    on the bf16 matrix cores; fp32 z is carried as bf16 hi + lo (~2^-17 per
    value). Small MFMA: z is carried as FP6 (E2M3) residual terms with a
    power-of-two scale per 32-value block, 4 terms for fp32 z up to B = 12
    (observed rel-L2 ~1e-6), 3 terms beyond (~4e-5), 2 terms for bf16 z
    (~8e-4, finer than a bf16 rounding of z)."""
    if algo == "valu":
        return 2e-5
    if algo == "mfma_large":
        return 2e-5 if zdtype == torch.bfloat16 else 1e-4
    if zdtype == torch.float32:
        return 3e-5 if B <= 12 else 2e-4      # 3 terms beyond B = 12
    return 3e-3


@pytest.mark.parametrize("algo", list(ALGOS))
@pytest.mark.parametrize("zdtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,L,B", SIGN_CASES)
def test_sign_gemm(lq, algo, zdtype, N, L, B):
    S, z, r = _sign_inputs(N, L, B, N + L + B, zdtype)
    packed = dev(rp.refpack(S))
    y = sign_gemm(lq, packed, dev(z, zdtype), B, N, L, dev(r), torch.float32, ALGOS[algo])
    want = ref.sign_matmul(S, z, r)
    err = rel_l2(host(y), want)
    assert err < sign_tol(algo, zdtype, B), err


@pytest.mark.parametrize("P", [2, 3, 5, 6, 7, 8])
@pytest.mark.parametrize("B", [1, 6, 13])
def test_sign_gemm_panels_per_workgroup(lq, P, B):
    """The small-batch product with P 16-row panels per workgroup (the plan
    takes the fewest that give at most one workgroup per compute unit: N =
    16 * 256 * P rows; at most 4 beyond 32 operand columns): two full tiles
    and a tail."""
    N, L = 16 * 256 * P, 1096
    S, z, r = _sign_inputs(N, L, B, 7 * P + B, torch.bfloat16)
    packed = dev(rp.refpack(S))
    y = sign_gemm(lq, packed, dev(z, torch.bfloat16), B, N, L, dev(r), torch.float32,
                  ALGOS["mfma_small"])
    want = ref.sign_matmul(S, z, r)
    err = rel_l2(host(y), want)
    assert err < sign_tol("mfma_small", torch.bfloat16, B), err


@pytest.mark.parametrize("algo", ["valu", "mfma_large"])
@pytest.mark.parametrize("B", [17, 33, 64, 100])
def test_sign_gemm_larger_batches(lq, algo, B):
    N, L = 80, 1544
    S, z, r = _sign_inputs(N, L, B, B, torch.bfloat16)
    y = sign_gemm(lq, dev(rp.refpack(S)), dev(z, torch.bfloat16), B, N, L, dev(r), torch.float32, ALGOS[algo])
    assert rel_l2(host(y), ref.sign_matmul(S, z, r)) < 2e-5


@pytest.mark.parametrize("algo", list(ALGOS))
def test_sign_gemm_bf16_output(lq, algo):
    N, L, B = 64, 2056, 4
    S, z, r = _sign_inputs(N, L, B, 99, torch.bfloat16)
    y = sign_gemm(lq, dev(rp.refpack(S)), dev(z, torch.bfloat16), B, N, L, dev(r), torch.bfloat16, ALGOS[algo])
    want = ref.sign_matmul(S, z, r)
    assert rel_l2(host(y), want) < 4e-3


@pytest.mark.parametrize("algo", list(ALGOS))
def test_sign_gemm_deterministic(lq, algo):
    N, L, B = 128, 9840, 4
    S, z, r = _sign_inputs(N, L, B, 5, torch.bfloat16)
    packed, zt, rt = dev(rp.refpack(S)), dev(z, torch.bfloat16), dev(r)
    y1 = sign_gemm(lq, packed, zt, B, N, L, rt, torch.float32, ALGOS[algo])
    y2 = sign_gemm(lq, packed, zt, B, N, L, rt, torch.float32, ALGOS[algo])
    assert torch.equal(y1, y2)


def test_sign_gemm_algorithms_agree_on_signs_only(lq):
    """All algorithms see the same packed bits: with z = one-hot columns the
    product returns the sign column itself, exactly."""
    N, L = 32, 1544
    S = _signs(11, N, L)
    cols = [0, 1, 31, 32, 127, 128, 511, 512, 1023, 1535, 1536, 1543]
    z = np.zeros((len(cols), L), dtype=np.float32)
    for i, j in enumerate(cols):
        z[i, j] = 1.0
    B = len(cols)
    for algo in ALGOS.values():
        y = sign_gemm(lq, dev(rp.refpack(S)), dev(z), B, N, L, dev(np.ones(N, np.float32)), torch.float32, algo)
        assert np.array_equal(host(y), S[:, cols].T.astype(np.float32)), algo
