"""lq_linear_multi: several layers on the same input (the gate and up
projections of a transformer MLP) in one preparation launch and one product
launch where the small-batch matrix-core path applies.

Each output must equal what lq_linear writes for that layer alone: bit for
bit where the grouped product splits the work among workgroups as the single
call does (few panels: one panel per workgroup either way), to fp32 rounding
where the panels per workgroup are chosen for both layers together, on:
* the Llama-3-8B gate and up shapes at batch 1 (d=10, D=24, K=4096,
  N=14336), bf16 x and y: 8 panels per workgroup instead of 4, so the
  per-wavefront partial sums differ; rel-L2 <= 1e-6 of fp32 y against the
  single calls, and the bf16 outputs agree but for a rounding step;
* small layers sharing K with different d, D, hb and N (grouped or run one
  after another, depending on whether their product plans match), batch 1-16,
  bf16 and fp32 x (fp32 x at B <= 16 runs the exact VALU product one layer
  after another), 2-4 layers;
* the oracle's operator on one grouped case (rel-L2 within the bf16 bound).
"""
import numpy as np
import pytest
import torch

from oracle import liftquant_ref as ref
from tests.gpu_util import DeviceLayer, dev, host, note, rel_l2, workspace
from workloads import make_layer_small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lq():
    import bit_matmul_amd
    assert torch.cuda.is_available()
    return bit_matmul_amd


def _multi(lq, layers, x, B, ydtype):
    ys = [torch.empty((B, l.N), dtype=ydtype, device="cuda") for l in layers]
    structs = [l.struct for l in layers]
    ws = workspace(lq, lq.lq_linear_multi_workspace_size(structs, B, x.dtype))
    note(f"lq_linear_multi n={len(layers)} B={B} x={x.dtype} "
         + " ".join(f"(N={l.N} d={l.d} D={l.D} hb={l.hb})" for l in layers))
    lq.lq_linear_multi(structs, x, B, ys, ws)
    torch.cuda.synchronize()
    return ys


def _check_identical(lq, layers, x, B, ydtype):
    ys = _multi(lq, layers, x, B, ydtype)
    for l, y in zip(layers, ys):
        y1 = l.linear(lq, x, B, ydtype)
        assert torch.equal(y.view(torch.int16) if ydtype == torch.bfloat16 else y.view(torch.int32),
                           y1.view(torch.int16) if ydtype == torch.bfloat16 else y1.view(torch.int32))
    return ys


def _check_close(lq, layers, x, B):
    """fp32 y within fp32 rounding of the single calls; bf16 y equal but for
    elements one rounding step apart."""
    ys = _multi(lq, layers, x, B, torch.float32)
    for l, y in zip(layers, ys):
        y1 = l.linear(lq, x, B, torch.float32)
        assert rel_l2(host(y), host(y1)) <= 1e-6
    yb = _multi(lq, layers, x, B, torch.bfloat16)
    for l, y in zip(layers, yb):
        y1 = l.linear(lq, x, B, torch.bfloat16)
        a, b = y.view(torch.int16).cpu().numpy().astype(np.int32), y1.view(torch.int16).cpu().numpy().astype(np.int32)
        assert np.abs(a - b).max() <= 1                  # adjacent bf16 codes at most
        assert (a != b).mean() < 0.01


@pytest.fixture(scope="module")
def gate_up(lq):
    N, K, d, D, hb = 14336, 4096, 10, 24, 1024
    return [DeviceLayer(make_layer_small(N, K, d, D, hb, seed=s, B_max=1, xdtype="bf16"), lq)
            for s in (701, 702)]


def test_gate_up_full_size(lq, gate_up):
    x = dev(np.random.default_rng(3).standard_normal((1, 4096)).astype(np.float32), torch.bfloat16)
    _check_close(lq, gate_up, x, 1)


SMALL = [
    # (K, [(N, d, D, hb), ...])
    (1024, [(64, 3, 8, 1024), (64, 3, 8, 1024)]),
    (1024, [(64, 3, 8, 1024), (96, 2, 4, 512), (32, 5, 16, 256)]),
    (2048, [(128, 10, 24, 1024), (128, 10, 24, 1024), (128, 10, 24, 1024), (128, 10, 24, 1024)]),
    (1536, [(48, 4, 8, 512), (48, 1, 2, 512)]),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("B", [1, 3, 16])
@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_small_layers_identical(lq, case, B, xdtype):
    K, shapes = SMALL[case]
    layers = [DeviceLayer(make_layer_small(N, K, d, D, hb, seed=100 * case + i, B_max=B,
                                           xdtype=xdtype), lq)
              for i, (N, d, D, hb) in enumerate(shapes)]
    xd = torch.bfloat16 if xdtype == "bf16" else torch.float32
    x = dev(np.random.default_rng(case + B).standard_normal((B, K)).astype(np.float32), xd)
    _check_identical(lq, layers, x, B, torch.float32)


def test_grouped_against_oracle(lq):
    K = 2048
    inps = [make_layer_small(64, K, 3, 8, 1024, seed=s, B_max=5, xdtype="bf16") for s in (11, 12)]
    layers = [DeviceLayer(i, lq) for i in inps]
    x = inps[0].x(5)
    xb = dev(x.astype(np.float32), torch.bfloat16)
    ys = _multi(lq, layers, xb, 5, torch.float32)
    xr = host(xb).astype(np.float64)
    for inp, y in zip(inps, ys):
        want = ref.linear(xr, inp.c, inp.spec.hb, inp.M, inp.signs(), inp.row_scale)
        assert rel_l2(host(y), want) < 1e-2


def test_errors(lq, gate_up):
    x = torch.zeros((1, 4096), dtype=torch.bfloat16, device="cuda")
    ys = [torch.empty((1, 14336), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    small = [l.struct for l in gate_up]
    with pytest.raises(lq.LQError):                   # no workspace
        lq.lq_linear_multi(small, x, 1, ys, None)
    with pytest.raises(ValueError):                   # one output per layer
        lq.lq_linear_multi(small, x, 1, ys[:1], None)
    with pytest.raises(lq.LQError):                   # more than LQ_MULTI_MAX layers
        lq.lq_linear_multi_workspace_size(small * 3, 1, torch.bfloat16)


def test_empty_layer_and_graph_replay(lq):
    """A layer with N = 0 is skipped; the grouped launches captured in a HIP
    graph replay to the eager result every time (eager work and
    synchronisation between the replays)."""
    K = 1024
    inps = [make_layer_small(64, K, 3, 8, 1024, seed=s, B_max=2, xdtype="bf16") for s in (31, 32)]
    layers = [DeviceLayer(i, lq) for i in inps]
    empty = lq.layer_struct(0, K, 3, 8, 1024, layers[0].packed, layers[0].M, layers[0].c, layers[0].r)
    x = dev(inps[0].x(2).astype(np.float32), torch.bfloat16)
    structs = [layers[0].struct, empty, layers[1].struct]
    ys = [torch.full((2, 64), -7.0, device="cuda"), torch.empty((2, 0), device="cuda"),
          torch.full((2, 64), -7.0, device="cuda")]
    ws = workspace(lq, lq.lq_linear_multi_workspace_size(structs, 2, torch.bfloat16))
    note("lq_linear_multi with an empty layer, then a graph of it")
    lq.lq_linear_multi(structs, x, 2, ys, ws)
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    for l, y in zip([layers[0], layers[1]], [eager[0], eager[2]]):
        assert torch.equal(y, l.linear(lq, x, 2, torch.float32))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lq.lq_linear_multi(structs, x, 2, ys, ws)
    for _ in range(3):
        ys[0].fill_(-1.0)
        ys[2].fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys[0], eager[0]) and torch.equal(ys[2], eager[2])
