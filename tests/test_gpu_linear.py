"""Parity of the whole decode operator (lq_linear) with the CPU oracle.

* Every layer of every workload at its full size and each of its batch
  sizes, in the launch configuration the benchmark times (lq_linear's own
  dispatch): sampled output rows, recomputed by the oracle one by one.
* The tiny 2.5-bit layer (fp32 activations) in full.
* Edge cases: empty batch, every batch size 1..17, K not a multiple of d,
  D = d with M = I, hb = 1, a single 16-row panel, D = 32 (the 2-bit LQ-32/16
  configuration), d = 1.
Tolerances: rel-L2 <= 1e-4 (fp32 activations), <= 1e-2 (bf16 activations).
"""
import numpy as np
import pytest
import torch

from oracle import liftquant_ref as ref
from tests.gpu_util import DEV, DeviceLayer, dev, host, note, rel_l2
from workloads import WORKLOADS, make_layer, make_layer_small

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


@pytest.fixture(scope="module")
def lq():
    import bit_matmul_amd
    assert torch.cuda.is_available()
    return bit_matmul_amd


def _xdtype(wl):
    return torch.float32 if wl.xdtype == "f32" else torch.bfloat16


def test_tiny_full(lq):
    wl = WORKLOADS["tiny"]
    spec = wl.layers[0]
    inp = make_layer(spec, wl)
    layer = DeviceLayer(inp, lq)
    x = inp.x(1)
    y = layer.linear(lq, dev(x), 1, torch.float32)
    want = ref.linear(x, inp.c, spec.hb, inp.M, inp.signs(), inp.row_scale)
    err = rel_l2(host(y), want)
    assert err < 1e-4, err
    assert err < 1e-5          # fp32 end to end: far inside the bar


FULL = [(w, i) for w in WORKLOADS for i in range(len(WORKLOADS[w].layers)) if w != "tiny"]


@pytest.mark.parametrize("wl_name,li", FULL, ids=[f"{w}-{WORKLOADS[w].layers[i].name}" for w, i in FULL])
def test_full_size_sampled_rows(lq, wl_name, li):
    wl = WORKLOADS[wl_name]
    spec = wl.layers[li]
    inp = make_layer(spec, wl)
    layer = DeviceLayer(inp, lq)
    xd = _xdtype(wl)
    rng = np.random.default_rng(spec.seed)
    rows = np.sort(rng.choice(spec.N, size=48, replace=False))
    rows[0], rows[-1] = 0, spec.N - 1
    for B in wl.batches:
        x = inp.x(B)
        for yd in (torch.float32, torch.bfloat16):
            y = host(layer.linear(lq, dev(x, xd), B, yd))
            bsel = np.arange(B) if B <= 64 else np.sort(rng.choice(B, 64, replace=False))
            want = ref.linear(x[bsel], inp.c, spec.hb, inp.M, inp.signs_rows(rows), inp.row_scale[rows])
            err = rel_l2(y[np.ix_(bsel, rows)], want)
            assert err < TOL[xd], (B, yd, err)
            assert np.all(np.isfinite(y))


EDGE = [
    # (N, K, d, D, hb, xdtype, label)
    (16, 64, 2, 8, 64, torch.float32, "single panel"),
    (32, 1037, 10, 24, 1, torch.float32, "K not a multiple of d, hb=1"),
    (48, 256, 4, 4, 256, torch.float32, "D = d"),
    (64, 4096, 16, 32, 1024, torch.bfloat16, "LQ-32/16 (2 bit)"),
    (32, 600, 1, 8, 8, torch.float32, "d = 1"),
    (16, 8192, 3, 8, 1024, torch.bfloat16, "2.67 bit ragged pad"),
    (80, 24, 8, 24, 8, torch.bfloat16, "LQ-24/8 (3 bit)"),
]


@pytest.mark.parametrize("N,K,d,D,hb,xd,label", EDGE, ids=[e[-1] for e in EDGE])
@pytest.mark.parametrize("B", [1, 2, 3, 5, 16, 17])
def test_edge_shapes(lq, N, K, d, D, hb, xd, label, B):
    inp = make_layer_small(N, K, d, D, hb, seed=N + K + d + D, B_max=17,
                           xdtype="f32" if xd == torch.float32 else "bf16")
    if label == "D = d":
        inp.M = np.eye(d, dtype=np.float32)
    layer = DeviceLayer(inp, lq)
    x = inp.x(B)
    y = layer.linear(lq, dev(x, xd), B, torch.float32)
    want = ref.linear(x, inp.c, hb, inp.M, inp.signs(), inp.row_scale)
    assert rel_l2(host(y), want) < TOL[xd]


def test_every_batch_size_small(lq):
    inp = make_layer_small(64, 2048, 10, 24, 1024, seed=77, B_max=17, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    for B in range(1, 18):
        x = inp.x(B)
        y = layer.linear(lq, dev(x, torch.bfloat16), B, torch.float32)
        want = ref.linear(x, inp.c, 1024, inp.M, inp.signs(), inp.row_scale)
        err = rel_l2(host(y), want)
        assert err < 1e-2, B
        if B <= 16:                # three FP6 terms per value; B = 17 rounds z to bf16
            assert err < 5e-4, (B, err)


def test_every_batch_size_small_fp32(lq):
    """fp32 activations, every batch size of the small-batch path: four FP6
    terms per value (three beyond B = 12) keep the operator within 2e-5
    (2e-4) of the oracle."""
    inp = make_layer_small(48, 3072, 10, 24, 128, seed=78, B_max=16, xdtype="f32")
    layer = DeviceLayer(inp, lq)
    for B in range(1, 17):
        x = inp.x(B)
        y = layer.linear(lq, dev(x), B, torch.float32)
        want = ref.linear(x, inp.c, 128, inp.M, inp.signs(), inp.row_scale)
        err = rel_l2(host(y), want)
        assert err < (2e-5 if B <= 12 else 2e-4), (B, err)


def test_empty_batch_is_noop(lq):
    inp = make_layer_small(16, 64, 2, 8, 64, seed=1, B_max=1)
    layer = DeviceLayer(inp, lq)
    y = torch.full((1, 16), 7.0, device=DEV)
    note("lq_linear B=0")
    lq.lq_linear(layer.struct, dev(inp.x(1)), 0, y, None)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_linear_deterministic(lq):
    wl = WORKLOADS["llama3_8b_mlp"]
    inp = make_layer(wl.layers[1], wl)
    layer = DeviceLayer(inp, lq)
    x = dev(inp.x(1), torch.bfloat16)
    y1 = layer.linear(lq, x, 1, torch.float32)
    y2 = layer.linear(lq, x, 1, torch.float32)
    assert torch.equal(y1, y2)
