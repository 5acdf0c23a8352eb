"""lq_linear_noalloc (no workspace, the library's own device scratch) against
lq_linear with a caller workspace, on the same inputs: bitwise equal outputs
(the same algorithm and kernels), and both within the oracle's tolerance.
Calls in a row share the scratch: a larger call, then a smaller one of
another algorithm, then the first again; a call whose workspace would exceed
the scratch is rejected on the host."""
import numpy as np
import pytest
import torch

from oracle import liftquant_ref as ref
from tests.gpu_util import DEV, DeviceLayer, dev, host, note, rel_l2
from workloads import make_layer_small

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


@pytest.fixture(scope="module")
def lq():
    import bit_matmul_amd
    assert torch.cuda.is_available()
    return bit_matmul_amd


# (N, K, d, D, hb, x dtype, B, the algorithm lq_linear runs)
CASES = [
    (1024, 8192, 10, 24, 1024, torch.bfloat16, 4, "MFMA_SMALL"),
    (512, 2048, 2, 5, 512, torch.float32, 1, "VALU"),
    (256, 1024, 3, 8, 1024, torch.bfloat16, 40, "WSPACE"),
]


def _run(lq, case, seed):
    N, K, d, D, hb, xd, B, algo = case
    inp = make_layer_small(N, K, d, D, hb, seed=seed, B_max=B,
                           xdtype="f32" if xd == torch.float32 else "bf16")
    layer = DeviceLayer(inp, lq)
    assert lq.lq_linear_algo(layer.struct, B, xd) == getattr(lq, "LQ_ALGO_" + algo)
    x = dev(inp.x(B), xd)
    want = layer.linear(lq, x, B, torch.float32)
    got = torch.full((B, N), float("nan"), dtype=torch.float32, device=DEV)
    note(f"lq_linear_noalloc N={N} K={K} d={d} D={D} B={B} x={xd} ({algo})")
    lq.lq_linear_noalloc(layer.struct, x, B, got)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"{algo}: differs from lq_linear"
    y_ref = ref.linear(inp.x(B), inp.c, hb, inp.M, inp.signs(), inp.row_scale)
    assert rel_l2(host(got), y_ref) < TOL[xd]


def test_noalloc_matches_lq_linear_in_sequence(lq):
    # a larger call, a smaller one, another algorithm, then the first again
    _run(lq, CASES[0], seed=5)
    _run(lq, CASES[1], seed=6)
    _run(lq, CASES[2], seed=7)
    _run(lq, CASES[0], seed=8)


def test_noalloc_rejects_calls_beyond_the_scratch(lq):
    N, K, d, D, hb, B = 16, 8192, 3, 8, 1024, 2048
    inp = make_layer_small(N, K, d, D, hb, seed=9, B_max=1, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    assert lq.lq_linear_workspace_size(layer.struct, B, torch.bfloat16) > lq.LQ_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, K), dtype=torch.bfloat16, device=DEV)
    y = torch.full((B, N), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(lq.LQError) as ei:
        lq.lq_linear_noalloc(layer.struct, x, B, y)
    assert ei.value.status == 2          # LQ_ERR_UNSUPPORTED, nothing enqueued
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
