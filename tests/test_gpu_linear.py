"""Parity of the whole decode operator (lq_linear) with the CPU oracle.

* Every layer of every workload at its full size and each of its batch
  sizes, in the launch configuration the benchmark times (lq_linear's own
  dispatch): every output row at every batch size (the oracle run over
  chunks of rows), and sampled rows with bf16 outputs too; at batch 1 also
  the Llama-3-70B gate and up layers through one lq_linear_multi call as the
  benchmark's decode step runs them. Besides rel-L2, every element must be
  within 10 x the tolerance of the output's RMS (a fault confined to a few
  workgroups would show there).
* The tiny 2.5-bit layer (fp32 activations) in full.
* The chunked small-batch product (batches beyond 1 whose records exceed
  LDS) on small shapes with partial, odd and even chunk counts and no tail,
  and through one grouped call.
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


def _rows_oracle(inp, spec, x, chunk=8192):
    """The oracle's operator for every output row, chunk by chunk of rows."""
    out = np.empty((x.shape[0], spec.N))
    for r0 in range(0, spec.N, chunk):
        rows = np.arange(r0, min(spec.N, r0 + chunk))
        out[:, rows] = ref.linear(x, inp.c, spec.hb, inp.M, inp.signs_rows(rows), inp.row_scale[rows])
    return out


def _check_all(got, want, tol):
    err = rel_l2(got, want)
    rms = float(np.sqrt(np.mean(want ** 2)))
    worst = float(np.max(np.abs(got.astype(np.float64) - want)))
    assert err < tol, err
    assert worst <= 10 * tol * rms, (worst, rms)
    assert np.all(np.isfinite(got))
    return err


@pytest.mark.parametrize("wl_name,li", FULL, ids=[f"{w}-{WORKLOADS[w].layers[i].name}" for w, i in FULL])
def test_full_size_every_row(lq, wl_name, li):
    """Every output row at every batch size of the workload (the oracle run
    once on the largest batch; a smaller batch is its leading rows)."""
    wl = WORKLOADS[wl_name]
    spec = wl.layers[li]
    inp = make_layer(spec, wl)
    layer = DeviceLayer(inp, lq)
    xd = _xdtype(wl)
    x = inp.x(max(wl.batches))
    want = _rows_oracle(inp, spec, x)
    for B in wl.batches:
        y = host(layer.linear(lq, dev(x[:B], xd), B, torch.float32))
        err = _check_all(y, want[:B], TOL[xd])
        if xd == torch.bfloat16 and B <= 16:
            assert err < 3e-3, (B, err)   # two FP6 terms per lifted value: ~8e-4 observed


def test_full_size_every_row_70b_gate_up_grouped(lq):
    """The benchmark's grouped call: gate and up of Llama-3-70B (two layers of
    the gate/up shape with their own weights) on one input, batch 1."""
    wl = WORKLOADS["llama3_70b"]
    spec = wl.layers[0]
    specs = [spec, type(spec)(spec.name + "_up", spec.K, spec.N, spec.d, spec.D, spec.hb, spec.seed + 1000)]
    inps = [make_layer(s, wl, B_max=1) for s in specs]
    layers = [DeviceLayer(i, lq) for i in inps]
    x = inps[0].x(1)
    xt = dev(x, torch.bfloat16)
    structs = [l.struct for l in layers]
    ys = [torch.empty((1, spec.N), dtype=torch.float32, device=DEV) for _ in layers]
    from tests.gpu_util import workspace
    ws = workspace(lq, lq.lq_linear_multi_workspace_size(structs, 1, torch.bfloat16))
    note("lq_linear_multi Llama-3-70B gate+up B=1")
    lq.lq_linear_multi(structs, xt, 1, ys, ws)
    torch.cuda.synchronize()
    for inp, s, y in zip(inps, specs, ys):
        _check_all(host(y), _rows_oracle(inp, s, x), 1e-2)


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


# Batch 1, bf16: records of at most 1 KB, more than 64 KB of them, so the
# small-batch product streams each tile's record with its slots.
STREAM = [
    # (N, K, d, D, hb, label): panels per workgroup as planned on 256 units
    (256, 16010, 10, 24, 2, "76 tiles with a 3-byte tail, 1 panel per workgroup"),
    (8192, 20000, 10, 24, 32, "94 tiles with a tail, 2 panels"),
    (10240, 16010, 10, 24, 2, "76 tiles with a tail, 3 panels"),
    (1040, 28672, 10, 24, 1024, "135 tiles, 65 panels"),
    (64, 40000, 2, 5, 64, "2.5 bit, 196 tiles: more records than LDS holds"),
]


@pytest.mark.parametrize("N,K,d,D,hb,label", STREAM, ids=[e[-1] for e in STREAM])
def test_streamed_records_batch1(lq, N, K, d, D, hb, label):
    inp = make_layer_small(N, K, d, D, hb, seed=N + K + 3, B_max=1, xdtype="bf16")
    L = -(-K // d) * D
    assert -(-L // 512) * 896 > 65536
    layer = DeviceLayer(inp, lq)
    x = inp.x(1)
    y = layer.linear(lq, dev(x, torch.bfloat16), 1, torch.float32)
    want = ref.linear(x, inp.c, hb, inp.M, inp.signs(), inp.row_scale)
    _check_all(host(y), want, 3e-3)


# Batches beyond 1 (bf16 x) whose activation records exceed LDS: the chunked
# small-batch product (loader wavefronts copy chunks of records while the
# compute wavefronts multiply). Chunks of W x tpc tiles: partial last chunks,
# odd and even chunk counts, a row with no tail tile, D = 5.
CHUNKED = [
    # (N, K, d, D, hb, B, label)
    (48, 2600, 10, 24, 8, 16, "B=16, 12 full tiles + tail: 3 chunks"),
    (32, 4480, 10, 24, 128, 16, "B=16, 21 tiles, no tail: 6 chunks, the last of one tile"),
    (64, 3008, 2, 5, 8, 16, "B=16, D=5, 14 tiles + tail: 4 chunks"),
    (16, 6840, 10, 24, 8, 5, "B=5, 32 tiles + tail: 4 chunks of 8"),
    (32, 9000, 10, 24, 8, 4, "B=4, 42 tiles + tail: 6 chunks, the last of two tiles"),
    (16, 18000, 10, 24, 16, 2, "B=2, 84 tiles + tail: 4 chunks of 24, the last of 12"),
]


def _rec_bytes(B):
    return -(-(804 * B) // 128) * 128        # two FP6 terms per batch row, bf16 x


@pytest.mark.parametrize("N,K,d,D,hb,B,label", CHUNKED, ids=[e[-1] for e in CHUNKED])
def test_chunked_records(lq, N, K, d, D, hb, B, label):
    L = -(-K // d) * D
    assert -(-L // 512) * _rec_bytes(B) > 128 * 1024      # records do not fit LDS
    inp = make_layer_small(N, K, d, D, hb, seed=N + K + B, B_max=B, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    x = inp.x(B)
    y = layer.linear(lq, dev(x, torch.bfloat16), B, torch.float32)
    want = ref.linear(x, inp.c, hb, inp.M, inp.signs(), inp.row_scale)
    _check_all(host(y), want, 3e-3)


def test_chunked_records_grouped(lq):
    """Two layers on one input through one lq_linear_multi call, B = 16, on
    the chunked product."""
    N, K, d, D, hb, B = 48, 2600, 10, 24, 8, 16
    inps = [make_layer_small(N, K, d, D, hb, seed=s, B_max=B, xdtype="bf16") for s in (5, 6)]
    layers = [DeviceLayer(i, lq) for i in inps]
    x = inps[0].x(B)
    ys = [torch.empty((B, N), dtype=torch.float32, device=DEV) for _ in layers]
    from tests.gpu_util import workspace
    structs = [l.struct for l in layers]
    ws = workspace(lq, lq.lq_linear_multi_workspace_size(structs, B, torch.bfloat16))
    note("lq_linear_multi chunked B=16")
    lq.lq_linear_multi(structs, dev(x, torch.bfloat16), B, ys, ws)
    torch.cuda.synchronize()
    for inp, y in zip(inps, ys):
        want = ref.linear(x, inp.c, hb, inp.M, inp.signs(), inp.row_scale)
        _check_all(host(y), want, 3e-3)


def test_every_batch_size_small(lq):
    inp = make_layer_small(64, 2048, 10, 24, 1024, seed=77, B_max=17, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    for B in range(1, 18):
        x = inp.x(B)
        y = layer.linear(lq, dev(x, torch.bfloat16), B, torch.float32)
        want = ref.linear(x, inp.c, 1024, inp.M, inp.signs(), inp.row_scale)
        err = rel_l2(host(y), want)
        assert err < 1e-2, B
        if B <= 16:                # two FP6 terms per value; B = 17 rounds z to bf16
            assert err < 3e-3, (B, err)


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
