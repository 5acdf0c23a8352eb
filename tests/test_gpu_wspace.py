"""Parity of the W-space large-batch product (LQ_ALGO_WSPACE) with the oracle.

The dense weights W[n][b d + i] = sum_e M[i][e] s[n][b][e] are rebuilt per
block from the packed signs and rounded to bf16; the transformed input is
rounded to bf16; the matrix cores reduce over d ceil(K/d) inputs. The bar is
the bf16 one, rel-L2 <= 1e-2, for bf16 activations (the only ones the path
takes).

* The prefill layers at their full size and batch (2048 rows), in the launch
  configuration the benchmark times: sampled output rows and batch rows,
  recomputed by the oracle one by one; and the whole output against the
  lifted large-batch product (both bf16-operand paths). (lq_linear's own
  dispatch takes this product for these layers; tests/test_gpu_linear.py
  compares its every output with the oracle's.)
* Small shapes spanning several tiles with a ragged tail: every batch size
  1..17 and 33, d = 1..4, D = 4 and 8, K not a multiple of d, hb = 1,
  bf16 and fp32 outputs, a single panel, many panels.
* Determinism, and an empty batch.
"""
import numpy as np
import pytest
import torch

from oracle import liftquant_ref as ref
from tests.gpu_util import DeviceLayer, dev, host, note, rel_l2
from workloads import WORKLOADS, make_layer, make_layer_small

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def lq():
    import bit_matmul_amd
    assert torch.cuda.is_available()
    return bit_matmul_amd


@pytest.mark.parametrize("li", [0, 1], ids=["sq", "wide"])
def test_prefill_full_size(lq, li):
    wl = WORKLOADS["prefill"]
    spec = wl.layers[li]
    inp = make_layer(spec, wl)
    layer = DeviceLayer(inp, lq)
    B = wl.batches[0]
    x = inp.x(B)
    xd = dev(x, torch.bfloat16)
    rng = np.random.default_rng(spec.seed + 5)
    rows = np.sort(rng.choice(spec.N, size=32, replace=False))
    rows[0], rows[-1] = 0, spec.N - 1
    bsel = np.sort(rng.choice(B, 48, replace=False))
    bsel[0], bsel[-1] = 0, B - 1
    want = ref.linear(x[bsel], inp.c, spec.hb, inp.M, inp.signs_rows(rows), inp.row_scale[rows])
    yw = layer.linear(lq, xd, B, torch.bfloat16, algo=lq.LQ_ALGO_WSPACE)
    got = host(yw)
    assert np.all(np.isfinite(got))
    err = rel_l2(got[np.ix_(bsel, rows)], want)
    assert err < TOL, err
    # the whole output against the lifted product (both round their operands
    # to bf16, at different places: each is within the bar of the oracle)
    yl = host(layer.linear(lq, xd, B, torch.bfloat16, algo=lq.LQ_ALGO_MFMA_LARGE))
    assert rel_l2(got, yl) < 2 * TOL


def test_ragged_batch_eight_tiles_per_workgroup(lq):
    """B = 2103 on the 8192 x 8192 layer: 132 batch tiles in workgroups of 8
    (the last group holds 4 real tiles, the last tile 7 real rows); sampled
    rows and batch rows, the last ones included."""
    wl = WORKLOADS["prefill"]
    spec = wl.layers[0]
    B = 2103
    inp = make_layer(spec, wl, B_max=B)
    layer = DeviceLayer(inp, lq)
    x = inp.x(B)
    rng = np.random.default_rng(2103)
    rows = np.sort(rng.choice(spec.N, size=24, replace=False))
    rows[0], rows[-1] = 0, spec.N - 1
    bsel = np.unique(np.concatenate([rng.choice(B, 24, replace=False), np.arange(B - 9, B)]))
    want = ref.linear(x[bsel], inp.c, spec.hb, inp.M, inp.signs_rows(rows), inp.row_scale[rows])
    y = host(layer.linear(lq, dev(x, torch.bfloat16), B, torch.float32, algo=lq.LQ_ALGO_WSPACE))
    assert np.all(np.isfinite(y))
    err = rel_l2(y[np.ix_(bsel, rows)], want)
    assert err < TOL, err


SMALL = [
    # (N, K, d, D, hb, label)
    (256, 2048, 3, 8, 1024, "prefill rate, 12 tiles + tail"),
    (128, 1037, 3, 8, 1, "K not a multiple of d, hb = 1"),
    (64, 1024, 4, 8, 512, "d = 4, no pad slot"),
    (96, 600, 1, 8, 8, "d = 1"),
    (48, 512, 2, 4, 512, "D = 4, d = 2"),
    (32, 1000, 4, 4, 8, "D = d = 4, M = I"),
    (16, 640, 3, 8, 128, "single panel"),
    (8192 // 16 * 16, 96, 2, 8, 32, "many panels, one tile"),
]


@pytest.mark.parametrize("N,K,d,D,hb,label", SMALL, ids=[s[-1] for s in SMALL])
@pytest.mark.parametrize("B", [1, 2, 5, 16, 17, 33])
def test_small_shapes(lq, N, K, d, D, hb, label, B):
    inp = make_layer_small(N, K, d, D, hb, seed=N + 3 * K + d + D, B_max=33, xdtype="bf16")
    if label.endswith("M = I"):
        inp.M = np.eye(d, dtype=np.float32)
    layer = DeviceLayer(inp, lq)
    x = inp.x(B)
    y = layer.linear(lq, dev(x, torch.bfloat16), B, torch.float32, algo=lq.LQ_ALGO_WSPACE)
    want = ref.linear(x, inp.c, hb, inp.M, inp.signs(), inp.row_scale)
    err = rel_l2(host(y), want)
    assert err < TOL, (label, B, err)


def test_bf16_output_every_batch(lq):
    inp = make_layer_small(256, 2048, 3, 8, 1024, seed=4242, B_max=40, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    for B in list(range(1, 18)) + [31, 40]:
        x = inp.x(B)
        y = layer.linear(lq, dev(x, torch.bfloat16), B, torch.bfloat16, algo=lq.LQ_ALGO_WSPACE)
        want = ref.linear(x, inp.c, 1024, inp.M, inp.signs(), inp.row_scale)
        err = rel_l2(host(y), want)
        assert err < TOL, (B, err)


def test_deterministic_and_empty(lq):
    inp = make_layer_small(512, 4096, 3, 8, 1024, seed=91, B_max=64, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    x = dev(inp.x(64), torch.bfloat16)
    y1 = layer.linear(lq, x, 64, torch.float32, algo=lq.LQ_ALGO_WSPACE)
    y2 = layer.linear(lq, x, 64, torch.float32, algo=lq.LQ_ALGO_WSPACE)
    assert torch.equal(y1, y2)
    note("lq_linear_ex W space, empty batch")
    y0 = layer.linear(lq, x[:0], 0, torch.float32, algo=lq.LQ_ALGO_WSPACE)
    assert y0.shape == (0, 512)
