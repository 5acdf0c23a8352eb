"""Parity of the lifted large-batch product (LQ_ALGO_MFMA_LARGE) with the
oracle, in every tiling it instantiates (tests/plan_cases.py: the CPU test
of the same list checks which tiling each shape gets), over the WHOLE output:

* lq_sign_gemm_ex on each shape: y = r * (S z) against the oracle's fp64
  sign product of the same (bf16-rounded or fp32) z;
* lq_linear_ex on the 8192 x 8192 prefill layer (d = 3, D = 8) at B = 2048
  (4 panels x 8 batch tiles per workgroup) and at a ragged B = 2103, every
  output against the oracle's dense route.

Bars. bf16 z is exact on the bf16 matrix cores and accumulation is fp32, so
the product is within fp32 rounding of the fp64 one (rel-L2 < 2e-5, every
element within 1e-4 of the output's RMS); fp32 z rides as a bf16 hi + lo
pair (about 2^-17 relative per value: rel-L2 < 1e-4, elements within 1e-3 of
the RMS). The whole operator with bf16 activations meets the bf16 bar of
rel-L2 1e-2 and every element within 10 x 1e-2 of the RMS.
"""
import numpy as np
import pytest
import torch

from oracle import liftquant_ref as ref
from tests.gpu_util import DEV, DeviceLayer, dev, host, note, rel_l2, sign_gemm
from tests.plan_cases import LARGE_PLAN_CASES, LARGE_SPLIT_CASES, case_id, split_case_id
from workloads import WORKLOADS, bf16_round, make_layer

pytestmark = pytest.mark.gpu

LARGE = 3


@pytest.fixture(scope="module")
def lq():
    import bit_matmul_amd
    assert torch.cuda.is_available()
    return bit_matmul_amd


def _check(got, want, rel, elem):
    err = rel_l2(got, want)
    rms = float(np.sqrt(np.mean(np.asarray(want, np.float64) ** 2)))
    worst = float(np.max(np.abs(np.asarray(got, np.float64) - want)))
    assert err < rel, f"rel-L2 {err}"
    assert worst <= elem * rms, f"max |diff| {worst} vs RMS {rms}"
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("case", LARGE_PLAN_CASES, ids=[case_id(c) for c in LARGE_PLAN_CASES])
def test_large_product_every_tiling(lq, case):
    N, L, B, zt, pw, jb = case
    zd = torch.bfloat16 if zt == "bf16" else torch.float32
    plan = lq.lq_sign_gemm_plan(B, N, L, zd, LARGE)
    assert (plan["panels"] // 4, plan["batch_rows"] // 16) == (pw, jb)
    rng = np.random.default_rng(N + 3 * L + 7 * B)
    S = np.where(rng.random((N, L), dtype=np.float32) < 0.5, -1, 1).astype(np.int8)
    z = rng.standard_normal((B, L)).astype(np.float32)
    if zd == torch.bfloat16:
        z = bf16_round(z)
    r = rng.uniform(0.5, 1.5, N).astype(np.float32)
    packed = torch.empty(N * L // 8, dtype=torch.uint8, device=DEV)
    note(f"lq_pack_signs N={N} L={L}")
    lq.lq_pack_signs(dev(S), N, L, 1, 1, packed)      # bit-exact packer (test_pack_bit_exact)
    torch.cuda.synchronize()
    y = sign_gemm(lq, packed, dev(z, zd), B, N, L, dev(r), torch.float32, LARGE)
    want = ref.sign_matmul(S, z, r)
    if zd == torch.bfloat16:
        _check(host(y), want, 2e-5, 1e-4)
    else:
        _check(host(y), want, 1e-4, 1e-3)


@pytest.mark.parametrize("case", LARGE_SPLIT_CASES, ids=[split_case_id(c) for c in LARGE_SPLIT_CASES])
def test_large_product_split_reduction(lq, case):
    """Reduction ranges added by the reduce kernel (fp32 partial sums in the
    workspace), bf16 and fp32 y, every output against the oracle."""
    N, L, B, zt, pw, jb, ks = case
    zd = torch.bfloat16 if zt == "bf16" else torch.float32
    plan = lq.lq_sign_gemm_plan(B, N, L, zd, LARGE)
    assert (plan["panels"] // 4, plan["batch_rows"] // 16, plan["ksplit"]) == (pw, jb, ks)
    rng = np.random.default_rng(N + 5 * L + 11 * B)
    S = np.where(rng.random((N, L), dtype=np.float32) < 0.5, -1, 1).astype(np.int8)
    z = rng.standard_normal((B, L)).astype(np.float32)
    if zd == torch.bfloat16:
        z = bf16_round(z)
    r = rng.uniform(0.5, 1.5, N).astype(np.float32)
    packed = torch.empty(N * L // 8, dtype=torch.uint8, device=DEV)
    note(f"lq_pack_signs N={N} L={L}")
    lq.lq_pack_signs(dev(S), N, L, 1, 1, packed)
    torch.cuda.synchronize()
    want = ref.sign_matmul(S, z, r)
    y = sign_gemm(lq, packed, dev(z, zd), B, N, L, dev(r), torch.float32, LARGE)
    if zd == torch.bfloat16:
        _check(host(y), want, 2e-5, 1e-4)
    else:
        _check(host(y), want, 1e-4, 1e-3)
    yb = sign_gemm(lq, packed, dev(z, zd), B, N, L, dev(r), torch.bfloat16, LARGE)
    _check(host(yb).astype(np.float64), want, 1e-2, 2e-2)


@pytest.mark.parametrize("B", [2048, 2103])
def test_large_linear_prefill_layer_every_output(lq, B):
    wl = WORKLOADS["prefill"]
    spec = wl.layers[0]                                   # 8192 -> 8192, d = 3, D = 8
    inp = make_layer(spec, wl, B_max=2048)
    layer = DeviceLayer(inp, lq)
    x = inp.x(2048)
    if B > 2048:                                         # ragged: more rows, same recipe
        rng = np.random.default_rng(B)
        x = np.concatenate([x, bf16_round(rng.standard_normal((B - 2048, spec.K)).astype(np.float32))])
    plan = lq.lq_linear_plan(layer.struct, B, torch.bfloat16, LARGE)
    assert (plan["panels"] // 4, plan["batch_rows"] // 16) == (4, 8)
    y = host(layer.linear(lq, dev(x, torch.bfloat16), B, torch.float32, algo=LARGE))
    want = ref.linear(x, inp.c, spec.hb, inp.M, inp.signs(), inp.row_scale)
    _check(y, want, 1e-2, 0.1)


def test_large_linear_wide_prefill_layer(lq):
    """The 8192 -> 28672 prefill layer on the lifted product (the tiling of
    the benchmark's `large` object: 4 panels x 8 batch tiles per wavefront
    group), every output row for 64 sampled batch rows, both ends included."""
    wl = WORKLOADS["prefill"]
    spec = wl.layers[1]                                   # 8192 -> 28672, d = 3, D = 8
    inp = make_layer(spec, wl, B_max=2048)
    layer = DeviceLayer(inp, lq)
    B = 2048
    x = inp.x(B)
    plan = lq.lq_linear_plan(layer.struct, B, torch.bfloat16, LARGE)
    assert (plan["panels"] // 4, plan["batch_rows"] // 16, plan["ksplit"]) == (4, 8, 1)
    y = host(layer.linear(lq, dev(x, torch.bfloat16), B, torch.bfloat16, algo=LARGE))
    rng = np.random.default_rng(5)
    bsel = np.sort(rng.choice(B, 64, replace=False))
    bsel[0], bsel[-1] = 0, B - 1
    want = np.empty((len(bsel), spec.N))
    for r0 in range(0, spec.N, 8192):
        rows = np.arange(r0, min(spec.N, r0 + 8192))
        want[:, rows] = ref.linear(x[bsel], inp.c, spec.hb, inp.M, inp.signs_rows(rows), inp.row_scale[rows])
    _check(y[bsel].astype(np.float64), want, 1e-2, 0.1)


def test_large_linear_fp32_activations(lq):
    """lq_linear's default for fp32 activations beyond batch 16: the lifted
    product on a bf16 hi + lo pair of z (two panels per wavefront, two batch
    tiles here), every output against the oracle at the fp32 bar."""
    from workloads import make_layer_small
    N, K, d, D, hb, B = 16384, 1024, 2, 5, 1024, 128
    inp = make_layer_small(N, K, d, D, hb, seed=17, B_max=B, xdtype="f32")
    layer = DeviceLayer(inp, lq)
    plan = lq.lq_linear_plan(layer.struct, B, torch.float32)
    assert plan["algo"] == LARGE
    assert (plan["panels"] // 4, plan["batch_rows"] // 16) == (2, 2)
    x = inp.x(B)
    y = host(layer.linear(lq, dev(x), B, torch.float32))
    want = ref.linear(x, inp.c, hb, inp.M, inp.signs(), inp.row_scale)
    _check(y, want, 1e-4, 1e-3)
