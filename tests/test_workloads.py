"""Seeded input generators (no GPU)."""
import numpy as np
import torch

from workloads import WORKLOADS, bf16_round, bf16_bits, make_layer_small, sign_bits_to_int8


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bf16_bits(x), ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(bf16_round(x), ref.float().numpy())


def test_draws_are_reproducible_and_shaped():
    a = make_layer_small(32, 100, 3, 8, 4, seed=5, B_max=3, xdtype="bf16", outlier_frac=0.05, outlier_gain=20)
    b = make_layer_small(32, 100, 3, 8, 4, seed=5, B_max=3, xdtype="bf16", outlier_frac=0.05, outlier_gain=20)
    assert np.array_equal(a.sign_bytes, b.sign_bytes) and np.array_equal(a.x_max, b.x_max)
    s = a.spec
    assert a.M.shape == (3, 8) and a.signs().shape == (32, s.Kb, 8)
    assert set(np.unique(a.signs())) == {-1, 1}
    assert np.array_equal(bf16_round(a.x_max), a.x_max)
    assert len(a.outliers) == 5
    assert np.array_equal(a.signs_rows(np.array([3, 7])), a.signs()[[3, 7]])


def test_sign_bits_unpack():
    by = np.array([0b00000101, 0xFF], dtype=np.uint8)
    s = sign_bits_to_int8(by, 1, 16)
    assert list(s[0, :8]) == [-1, 1, -1, 1, 1, 1, 1, 1] and all(s[0, 8:] == -1)


def test_workload_shapes_fit_layout():
    for wl in WORKLOADS.values():
        for l in wl.layers:
            assert l.N % 16 == 0 and l.L % 8 == 0 and l.K % l.hb == 0
