"""Parity of the one-launch decode (lq_linear_ex with LQ_ALGO_FUSED) with the
CPU oracle and with the two-launch small-batch path, through the C ABI.

* Every layer of every workload at full size, at each batch size where the
  one-launch decode applies, bf16 and fp32 activations: sampled output rows
  recomputed by the oracle one by one.
* Same results as the two-launch path (MFMA_SMALL) up to fp32 summation
  order: both carry the lifted activations as the same FP6 terms.
* Ragged shapes: only a tail tile (L < 512), no tail (L % 512 == 0), K not a
  multiple of d, hb = 1, d = 1, D = d with M = I, one 16-row panel.
* One zero-filled workspace reused by many calls of different layers (the
  control words advance an epoch per launch), graph replays, determinism,
  and the error word staying clear (lq_workspace_status).
* The failure path, forced from the host (lq_debug_fused_timeout: the
  loaders wait for a publication no producer makes and give up after a few
  polls, every kernel still running to its end): lq_workspace_status reports
  LQ_ERR_DEVICE; after lq_workspace_init the next calls are right again.
Tolerances (relative L2): fp32 x 2e-5 (four FP6 terms), bf16 x 3e-3 (two: ~8e-4
observed, finer than rounding z to bf16).
"""
import numpy as np
import pytest
import torch

from oracle import liftquant_ref as ref
from tests.gpu_util import DEV, DeviceLayer, control_error, dev, host, note, rel_l2, workspace
from workloads import WORKLOADS, make_layer, make_layer_small

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 2e-5, torch.bfloat16: 3e-3}


@pytest.fixture(scope="module")
def lq():
    import bit_matmul_amd
    assert torch.cuda.is_available()
    return bit_matmul_amd


def _fused_ok(lq, layer, B, xd):
    try:
        lq.lq_linear_workspace_size_ex(layer.struct, B, xd, lq.LQ_ALGO_FUSED)
        return True
    except lq.LQError as e:
        assert e.status == 2, e          # UNSUPPORTED, nothing else
        return False


FULL = [(w, i) for w in WORKLOADS for i in range(len(WORKLOADS[w].layers)) if w != "tiny"]


@pytest.mark.parametrize("wl_name,li", FULL, ids=[f"{w}-{WORKLOADS[w].layers[i].name}" for w, i in FULL])
def test_fused_full_size_sampled_rows(lq, wl_name, li):
    wl = WORKLOADS[wl_name]
    spec = wl.layers[li]
    inp = make_layer(spec, wl, B_max=5)
    layer = DeviceLayer(inp, lq)
    rng = np.random.default_rng(spec.seed + 1)
    rows = np.sort(rng.choice(spec.N, size=48, replace=False))
    rows[0], rows[-1] = 0, spec.N - 1
    ran = 0
    for B in (1, 2, 3, 4, 5):
        x = inp.x(B)
        for xd in (torch.bfloat16, torch.float32):
            if not _fused_ok(lq, layer, B, xd):
                continue
            y = host(layer.linear(lq, dev(x, xd), B, torch.float32, algo=lq.LQ_ALGO_FUSED))
            want = ref.linear(x, inp.c, spec.hb, inp.M, inp.signs_rows(rows), inp.row_scale[rows])
            err = rel_l2(y[:, rows], want)
            assert err < TOL[xd], (B, xd, err)
            assert np.all(np.isfinite(y))
            ran += 1
    assert ran > 0 or spec.K * spec.D // spec.d > 512 * 256


def test_fused_batch1_applies_on_every_full_size_layer(lq):
    """Batch 1 with bf16 activations is the decode the one launch is for:
    every full-size layer qualifies, with a workspace no larger than the
    two-launch path's (which may also hold partial row sums)."""
    for wl_name, li in FULL:
        wl = WORKLOADS[wl_name]
        s = wl.layers[li]
        st = lq.layer_struct(s.N, s.K, s.d, s.D, s.hb, *(torch.empty(16, device=DEV),) * 4)
        a = lq.lq_linear_workspace_size_ex(st, 1, torch.bfloat16, lq.LQ_ALGO_MFMA_SMALL)
        f = lq.lq_linear_workspace_size_ex(st, 1, torch.bfloat16, lq.LQ_ALGO_FUSED)
        assert 0 < f <= a, (wl_name, s.name)


@pytest.mark.parametrize("xd", [torch.bfloat16, torch.float32])
def test_fused_matches_two_launch(lq, xd):
    inp = make_layer_small(2048, 4096, 10, 24, 1024, seed=91, B_max=4,
                           xdtype="bf16" if xd == torch.bfloat16 else "f32")
    layer = DeviceLayer(inp, lq)
    for B in (1, 2, 3, 4):
        x = dev(inp.x(B), xd)
        yf = host(layer.linear(lq, x, B, torch.float32, algo=lq.LQ_ALGO_FUSED))
        ys = host(layer.linear(lq, x, B, torch.float32, algo=lq.LQ_ALGO_MFMA_SMALL))
        assert rel_l2(yf, ys) < 2e-6, B
        want = ref.linear(inp.x(B), inp.c, 1024, inp.M, inp.signs(), inp.row_scale)
        assert rel_l2(yf, want) < TOL[xd]


EDGE = [
    # (N, K, d, D, hb, label)
    (16, 64, 2, 8, 64, "single panel, tail only"),
    (160, 1037, 10, 24, 1, "K not a multiple of d, hb=1"),
    (48, 256, 4, 4, 256, "D = d, tail only"),
    (512, 4096, 16, 32, 1024, "LQ-32/16, no tail"),
    (320, 600, 1, 8, 8, "d = 1"),
    (1024, 8192, 3, 8, 1024, "2.67 bit ragged pad"),
    (80, 24, 8, 24, 8, "LQ-24/8 one block row"),
    (1024, 2560, 5, 16, 512, "16 full tiles, no tail"),
    (512, 2600, 10, 24, 8, "ragged tail after 12 tiles"),
]


@pytest.mark.parametrize("N,K,d,D,hb,label", EDGE, ids=[e[-1] for e in EDGE])
@pytest.mark.parametrize("xd", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_fused_edge_shapes(lq, N, K, d, D, hb, label, xd):
    inp = make_layer_small(N, K, d, D, hb, seed=N + K + d + D + 5, B_max=5,
                           xdtype="f32" if xd == torch.float32 else "bf16")
    if label.startswith("D = d"):
        inp.M = np.eye(d, dtype=np.float32)
    layer = DeviceLayer(inp, lq)
    ran = 0
    for B in (1, 2, 3, 4, 5):
        if not _fused_ok(lq, layer, B, xd):
            continue
        x = inp.x(B)
        y = layer.linear(lq, dev(x, xd), B, torch.float32, algo=lq.LQ_ALGO_FUSED)
        want = ref.linear(x, inp.c, hb, inp.M, inp.signs(), inp.row_scale)
        assert rel_l2(host(y), want) < TOL[xd], B
        ran += 1
    assert ran > 0


def test_fused_shared_workspace_many_calls(lq):
    """One workspace, zero-filled once, serving interleaved calls of three
    layers of different geometry (and of the two-launch path) for several
    rounds: every call must see only its own launch's published operand."""
    shapes = [(512, 2048, 10, 24, 1024), (2048, 5120, 10, 24, 1024), (1024, 1024, 5, 16, 256)]
    layers, inps = [], []
    for i, (N, K, d, D, hb) in enumerate(shapes):
        inp = make_layer_small(N, K, d, D, hb, seed=200 + i, B_max=3, xdtype="bf16")
        inps.append(inp)
        layers.append(DeviceLayer(inp, lq))
    nbytes = max(lq.lq_linear_workspace_size_ex(l.struct, 3, torch.bfloat16, a)
                 for l in layers for a in (lq.LQ_ALGO_FUSED, lq.LQ_ALGO_MFMA_SMALL))
    ws = workspace(lq, nbytes)
    rng = np.random.default_rng(5)
    note("shared workspace: 3 layers x 4 rounds, fused and two-launch interleaved")
    for rnd in range(4):
        for li, (layer, inp) in enumerate(zip(layers, inps)):
            B = 1 + (rnd + li) % 3
            x = (rng.standard_normal((B, layer.K)).astype(np.float32))
            xb = dev(x, torch.bfloat16)
            algo = lq.LQ_ALGO_FUSED if (rnd + li) % 4 != 3 else lq.LQ_ALGO_MFMA_SMALL
            y = torch.empty((B, layer.N), dtype=torch.float32, device=DEV)
            lq.lq_linear_ex(layer.struct, xb, B, y, algo, ws)
            torch.cuda.synchronize()
            want = ref.linear(host(xb).astype(np.float32), inp.c, layer.hb, inp.M, inp.signs(),
                              inp.row_scale)
            assert rel_l2(host(y), want) < TOL[torch.bfloat16], (rnd, li, algo)
    assert control_error(lq, ws) == 0


def test_fused_graph_replay(lq):
    """A captured one-launch decode replays correctly: the control words are
    reset by the kernel itself (no memset node), each replay checked against
    the eager result, with eager work of the same workspace in between."""
    inp = make_layer_small(2048, 4096, 10, 24, 1024, seed=301, B_max=2, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    B = 2
    nbytes = lq.lq_linear_workspace_size_ex(layer.struct, B, torch.bfloat16, lq.LQ_ALGO_FUSED)
    ws = workspace(lq, nbytes)
    x = dev(inp.x(B), torch.bfloat16)
    y = torch.empty((B, layer.N), dtype=torch.float32, device=DEV)
    lq.lq_linear_ex(layer.struct, x, B, y, lq.LQ_ALGO_FUSED, ws)      # warm (LDS attribute set)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    note("capture one-launch decode")
    with torch.cuda.graph(g, stream=s):
        lq.lq_linear_ex(layer.struct, x, B, y, lq.LQ_ALGO_FUSED, ws, stream=s)
    rng = np.random.default_rng(9)
    for rep in range(4):
        xn = rng.standard_normal((B, layer.K)).astype(np.float32)
        x.copy_(dev(xn, torch.bfloat16))
        note(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        y_eager = torch.empty_like(y)
        lq.lq_linear_ex(layer.struct, x, B, y_eager, lq.LQ_ALGO_FUSED, ws)
        torch.cuda.synchronize()
        assert torch.equal(got, y_eager), rep
        want = ref.linear(host(x).astype(np.float32), inp.c, 1024, inp.M, inp.signs(), inp.row_scale)
        assert rel_l2(host(got), want) < TOL[torch.bfloat16]
    assert control_error(lq, ws) == 0


def test_fused_deterministic(lq):
    wl = WORKLOADS["llama3_8b_mlp"]
    inp = make_layer(wl.layers[1], wl, B_max=1)
    layer = DeviceLayer(inp, lq)
    x = dev(inp.x(1), torch.bfloat16)
    y1 = layer.linear(lq, x, 1, torch.bfloat16, algo=lq.LQ_ALGO_FUSED)
    y2 = layer.linear(lq, x, 1, torch.bfloat16, algo=lq.LQ_ALGO_FUSED)
    assert torch.equal(y1, y2)


# ---- one launch without communication (LQ_ALGO_FUSED_LOCAL): batch 1


def _local_ok(lq, layer, xd):
    try:
        lq.lq_linear_workspace_size_ex(layer.struct, 1, xd, lq.LQ_ALGO_FUSED_LOCAL)
        return True
    except lq.LQError as e:
        assert e.status == 2, e
        return False


def test_local_full_size_gate_up(lq):
    """Llama-3-8B gate/up (K = 4096, L = 9840): sampled rows against the
    oracle, and the whole output against the two-launch path."""
    wl = WORKLOADS["llama3_8b_mlp"]
    spec = wl.layers[0]
    inp = make_layer(spec, wl, B_max=1)
    layer = DeviceLayer(inp, lq)
    assert _local_ok(lq, layer, torch.bfloat16)
    rng = np.random.default_rng(spec.seed + 2)
    rows = np.sort(rng.choice(spec.N, size=64, replace=False))
    for xd in (torch.bfloat16, torch.float32):
        x = dev(inp.x(1), xd)
        yl = host(layer.linear(lq, x, 1, torch.float32, algo=lq.LQ_ALGO_FUSED_LOCAL))
        ys = host(layer.linear(lq, x, 1, torch.float32, algo=lq.LQ_ALGO_MFMA_SMALL))
        assert rel_l2(yl, ys) < 2e-6, xd
        want = ref.linear(inp.x(1), inp.c, spec.hb, inp.M, inp.signs_rows(rows), inp.row_scale[rows])
        assert rel_l2(yl[:, rows], want) < TOL[xd], xd


LOCAL = [
    # (N, K, d, D, hb, label)
    (128, 1024, 10, 24, 1024, "3 tiles, ragged tail"),
    (256, 2048, 4, 8, 512, "8 full tiles, no tail"),
    (64, 1037, 10, 24, 1, "K not a multiple of d, hb=1"),
    (8200 // 8 * 8 - 8, 512, 2, 5, 512, "1280 columns, many panels"),
    (96, 600, 1, 8, 8, "d = 1"),
    (48, 8192, 16, 16, 1024, "K = 8192, D = d, 16 full tiles"),
    (40 * 16, 4096, 10, 24, 1024, "partial last workgroup (40 panels)"),
    (16, 640, 10, 16, 128, "one panel"),
]


@pytest.mark.parametrize("N,K,d,D,hb,label", LOCAL, ids=[e[-1] for e in LOCAL])
@pytest.mark.parametrize("xd", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_local_shapes(lq, N, K, d, D, hb, label, xd):
    inp = make_layer_small(N, K, d, D, hb, seed=N + K + d + D + 11, B_max=1,
                           xdtype="f32" if xd == torch.float32 else "bf16")
    if label.startswith("K = 8192, D = d"):
        inp.M = np.eye(d, dtype=np.float32)
    layer = DeviceLayer(inp, lq)
    assert _local_ok(lq, layer, xd), label
    x = dev(inp.x(1), xd)
    y = host(layer.linear(lq, x, 1, torch.float32, algo=lq.LQ_ALGO_FUSED_LOCAL))
    want = ref.linear(inp.x(1), inp.c, hb, inp.M, inp.signs(), inp.row_scale)
    assert rel_l2(y, want) < TOL[xd]
    ys = host(layer.linear(lq, x, 1, torch.float32, algo=lq.LQ_ALGO_MFMA_SMALL))
    assert rel_l2(y, ys) < 2e-6


def test_local_bf16_output_and_determinism(lq):
    inp = make_layer_small(512, 4096, 10, 24, 1024, seed=404, B_max=1, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    x = dev(inp.x(1), torch.bfloat16)
    y1 = layer.linear(lq, x, 1, torch.bfloat16, algo=lq.LQ_ALGO_FUSED_LOCAL)
    y2 = layer.linear(lq, x, 1, torch.bfloat16, algo=lq.LQ_ALGO_FUSED_LOCAL)
    assert torch.equal(y1, y2)
    want = ref.linear(inp.x(1), inp.c, 1024, inp.M, inp.signs(), inp.row_scale)
    assert rel_l2(host(y1), want) < 5e-3          # bf16 output rounding


# ---- one launch split over the reduction (LQ_ALGO_FUSED_SPLIT): batch 1


@pytest.mark.parametrize("li", [0, 1], ids=["gate_up", "down"])
def test_split_full_size(lq, li):
    """Llama-3-8B gate/up and down at full size: sampled rows against the
    oracle, the whole output against the two-launch path, and a second call
    on the same workspace (the tickets reset themselves)."""
    wl = WORKLOADS["llama3_8b_mlp"]
    spec = wl.layers[li]
    inp = make_layer(spec, wl)
    layer = DeviceLayer(inp, lq)
    rng = np.random.default_rng(spec.seed + 9)
    rows = np.sort(rng.choice(spec.N, size=48, replace=False))
    rows[0], rows[-1] = 0, spec.N - 1
    x = dev(inp.x(1), torch.bfloat16)
    nbytes = lq.lq_linear_workspace_size_ex(layer.struct, 1, torch.bfloat16, lq.LQ_ALGO_FUSED_SPLIT)
    ws = workspace(lq, nbytes)
    outs = []
    for _ in range(2):
        y = torch.empty((1, spec.N), dtype=torch.float32, device="cuda")
        note(f"lq_linear_ex FUSED_SPLIT N={spec.N} K={spec.K}")
        lq.lq_linear_ex(layer.struct, x, 1, y, lq.LQ_ALGO_FUSED_SPLIT, ws)
        torch.cuda.synchronize()
        outs.append(host(y))
    assert np.array_equal(outs[0], outs[1])
    ys = host(layer.linear(lq, x, 1, torch.float32, algo=lq.LQ_ALGO_MFMA_SMALL))
    assert rel_l2(outs[0], ys) < 2e-6
    want = ref.linear(inp.x(1), inp.c, spec.hb, inp.M, inp.signs_rows(rows), inp.row_scale[rows])
    assert rel_l2(outs[0][:, rows], want) < 1e-2


SPLIT = [
    # (N, K, d, D, hb, label)
    (128, 1024, 10, 24, 1024, "3 tiles, ragged tail"),
    (256, 2048, 4, 8, 512, "8 full tiles, no tail"),
    (64, 1037, 10, 24, 1, "K not a multiple of d, hb=1"),
    (8200 // 8 * 8 - 8, 512, 2, 5, 512, "1280 columns, many panels"),
    (96, 600, 1, 8, 8, "d = 1"),
    (48, 8192, 16, 16, 1024, "K = 8192, D = d, 16 full tiles"),
    (40 * 16, 4096, 10, 24, 1024, "partial last panel group (40 panels)"),
    (16, 640, 10, 16, 128, "one panel"),
    (32, 14336, 10, 24, 1024, "long rows (68 tiles)"),
    (64, 2600, 3, 8, 8, "tail-only last group"),
]


@pytest.mark.parametrize("N,K,d,D,hb,label", SPLIT, ids=[e[-1] for e in SPLIT])
@pytest.mark.parametrize("xd", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_split_shapes(lq, N, K, d, D, hb, label, xd):
    inp = make_layer_small(N, K, d, D, hb, seed=N + K + d + D + 13, B_max=1,
                           xdtype="f32" if xd == torch.float32 else "bf16")
    if label.startswith("K = 8192, D = d"):
        inp.M = np.eye(d, dtype=np.float32)
    layer = DeviceLayer(inp, lq)
    x = dev(inp.x(1), xd)
    y = host(layer.linear(lq, x, 1, torch.float32, algo=lq.LQ_ALGO_FUSED_SPLIT))
    want = ref.linear(inp.x(1), inp.c, hb, inp.M, inp.signs(), inp.row_scale)
    assert rel_l2(y, want) < TOL[xd]
    ys = host(layer.linear(lq, x, 1, torch.float32, algo=lq.LQ_ALGO_MFMA_SMALL))
    assert rel_l2(y, ys) < 2e-6


def test_split_bf16_output_and_shared_workspace(lq):
    """bf16 output, and one workspace shared by interleaved calls of two
    layers and of the other algorithms."""
    a = make_layer_small(512, 4096, 10, 24, 1024, seed=405, B_max=4, xdtype="bf16")
    b = make_layer_small(256, 2048, 3, 8, 512, seed=406, B_max=4, xdtype="bf16")
    la, lb = DeviceLayer(a, lq), DeviceLayer(b, lq)
    xa, xb = dev(a.x(1), torch.bfloat16), dev(b.x(1), torch.bfloat16)
    algos = [lq.LQ_ALGO_FUSED_SPLIT, lq.LQ_ALGO_MFMA_SMALL, lq.LQ_ALGO_FUSED_SPLIT]
    need = max(lq.lq_linear_workspace_size_ex(l.struct, 1, torch.bfloat16, al)
               for l in (la, lb) for al in algos)
    ws = workspace(lq, need)
    ref_a = ref.linear(a.x(1), a.c, 1024, a.M, a.signs(), a.row_scale)
    ref_b = ref.linear(b.x(1), b.c, 512, b.M, b.signs(), b.row_scale)
    first = {}
    for it in range(3):
        for name, l, x, want in (("a", la, xa, ref_a), ("b", lb, xb, ref_b)):
            for al in algos:
                y = torch.empty((1, l.N), dtype=torch.bfloat16, device="cuda")
                note(f"shared workspace it={it} layer={name} algo={al}")
                lq.lq_linear_ex(l.struct, x, 1, y, al, ws)
                torch.cuda.synchronize()
                got = host(y)
                assert rel_l2(got, want) < 5e-3
                if al == lq.LQ_ALGO_FUSED_SPLIT:
                    if name in first:
                        assert np.array_equal(got, first[name])
                    first[name] = got
    assert control_error(lq, ws) == 0


def test_split_graph_replay(lq):
    inp = make_layer_small(1024, 4096, 10, 24, 1024, seed=407, B_max=1, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    x = dev(inp.x(1), torch.bfloat16)
    need = lq.lq_linear_workspace_size_ex(layer.struct, 1, torch.bfloat16, lq.LQ_ALGO_FUSED_SPLIT)
    ws = workspace(lq, need)
    y = torch.empty((1, inp.spec.N), dtype=torch.float32, device="cuda")
    lq.lq_linear_ex(layer.struct, x, 1, y, lq.LQ_ALGO_FUSED_SPLIT, ws)
    torch.cuda.synchronize()
    eager = host(y).copy()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            lq.lq_linear_ex(layer.struct, x, 1, y, lq.LQ_ALGO_FUSED_SPLIT, ws, stream=s)
    torch.cuda.synchronize()
    for i in range(4):
        y.zero_()
        note(f"split graph replay {i}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), eager)
        lq.lq_linear_ex(layer.struct, x, 1, y, lq.LQ_ALGO_MFMA_SMALL,
                        workspace(lq, lq.lq_linear_workspace_size_ex(layer.struct, 1, torch.bfloat16,
                                                                     lq.LQ_ALGO_MFMA_SMALL)))
        torch.cuda.synchronize()


def test_fused_failure_is_reported(lq):
    inp = make_layer_small(512, 4096, 10, 24, 1024, seed=91, B_max=1, xdtype="bf16")
    layer = DeviceLayer(inp, lq)
    x = dev(inp.x(1), torch.bfloat16)
    nbytes = lq.lq_linear_workspace_size_ex(layer.struct, 1, torch.bfloat16, lq.LQ_ALGO_FUSED)
    ws = workspace(lq, nbytes)
    y = torch.empty((1, 512), dtype=torch.float32, device=DEV)
    lq.lq_linear_ex(layer.struct, x, 1, y, lq.LQ_ALGO_FUSED, ws)
    assert lq.lq_workspace_status(ws) == 0
    note("lq_linear_ex FUSED with the forced give-up (test aid)")
    lq.lq_debug_fused_timeout(True)
    try:
        lq.lq_linear_ex(layer.struct, x, 1, y, lq.LQ_ALGO_FUSED, ws)
        lq.lq_linear_ex(layer.struct, x, 1, y, lq.LQ_ALGO_FUSED, ws)
    finally:
        lq.lq_debug_fused_timeout(False)
    assert lq.lq_workspace_status(ws) == lq.LQ_ERR_DEVICE
    assert lq.lq_workspace_status(ws) == lq.LQ_ERR_DEVICE     # stays set
    lq.lq_workspace_init(ws)
    assert lq.lq_workspace_status(ws) == 0
    for _ in range(3):                                        # the control words are consistent
        lq.lq_linear_ex(layer.struct, x, 1, y, lq.LQ_ALGO_FUSED, ws)
        torch.cuda.synchronize()
        assert lq.lq_workspace_status(ws) == 0
        want = ref.linear(inp.x(1), inp.c, 1024, inp.M, inp.signs(), inp.row_scale)
        assert rel_l2(host(y), want) < TOL[torch.bfloat16]
