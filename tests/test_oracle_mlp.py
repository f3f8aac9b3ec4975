"""Pins for the GeLU-MLP half of the oracle (CPU only)."""
import os

import numpy as np
import pytest

from oracle import (brute_mlp_forward, gelu, gelu_grad, mlp_backward, mlp_forward,
                    mlp_forward_rows)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape, sigma=1.0):
    return sigma * np.random.default_rng(seed).standard_normal(shape)


def load_gelu_points():
    pts = []
    with open(os.path.join(GOLDEN, "gelu_points.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                pts.append([float(x) for x in line.split()])
    return np.array(pts)


def test_gelu_closed_form_points():
    pts = load_gelu_points()
    np.testing.assert_allclose(gelu(pts[:, 0]), pts[:, 1], rtol=0, atol=2e-16)
    np.testing.assert_allclose(gelu_grad(pts[:, 0]), pts[:, 2], rtol=0, atol=4e-16)


def test_gelu_identities():
    x = np.linspace(-6, 6, 241)
    np.testing.assert_allclose(gelu(x) - gelu(-x), x, rtol=0, atol=1e-14)
    np.testing.assert_allclose(gelu_grad(x) + gelu_grad(-x), 1.0, rtol=0, atol=1e-14)
    # derivative by central differences
    h = 1e-6
    np.testing.assert_allclose((gelu(x + h) - gelu(x - h)) / (2 * h), gelu_grad(x),
                               rtol=0, atol=1e-8)


def test_brute_force_forward():
    a, bt, c = rnd(1, 5, 4), rnd(2, 6, 4), rnd(3, 6, 3)
    np.testing.assert_allclose(mlp_forward(a, bt, c, 0.7), brute_mlp_forward(a, bt, c, 0.7),
                               rtol=0, atol=1e-13)


def test_against_torch_float64():
    torch = pytest.importorskip("torch")
    a, bt, c, do = rnd(4, 33, 16), rnd(5, 40, 16), rnd(6, 40, 24), rnd(7, 33, 24)
    scale = 0.8
    o = mlp_forward(a, bt, c, scale, block_rows=7)
    da, dbt, dc = mlp_backward(a, bt, c, do, scale, block_rows=7)
    ta, tb, tc = (torch.tensor(x, requires_grad=True) for x in (a, bt, c))
    to = torch.nn.functional.gelu(scale * ta @ tb.T, approximate="none") @ tc
    to.backward(torch.tensor(do))
    for x, y in ((o, to), (da, ta.grad), (dbt, tb.grad), (dc, tc.grad)):
        np.testing.assert_allclose(x, y.detach().numpy(), rtol=0, atol=1e-12)


def test_finite_differences():
    a, bt, c, do = rnd(8, 4, 3), rnd(9, 5, 3), rnd(10, 5, 2), rnd(11, 4, 2)
    scale = 1.3
    grads = mlp_backward(a, bt, c, do, scale)
    h = 1e-6

    def loss(*x):
        return float(np.sum(mlp_forward(*x, scale) * do))

    base = [a, bt, c]
    for which, g in enumerate(grads):
        for idx in np.ndindex(base[which].shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx)


def test_zero_weights_special_case():
    a, c, do = rnd(12, 9, 6), rnd(13, 7, 5), rnd(14, 9, 5)
    bt = np.zeros((7, 6))
    scale = 0.9
    o = mlp_forward(a, bt, c, scale)
    da, dbt, dc = mlp_backward(a, bt, c, do, scale)
    assert np.all(o == 0) and np.all(dc == 0) and np.all(da == 0)
    # GeLU'(0) = 1/2, so dBt = scale/2 * (dO C^T)^T A
    np.testing.assert_allclose(dbt, 0.5 * scale * (do @ c.T).T @ a, rtol=0, atol=1e-13)


def test_linear_in_c_and_identity():
    a, bt, c, do = rnd(15, 11, 8), rnd(16, 13, 8), rnd(17, 13, 4), rnd(18, 11, 4)
    o = mlp_forward(a, bt, c, 1.0)
    np.testing.assert_allclose(mlp_forward(a, bt, 2.5 * c, 1.0), 2.5 * o, rtol=1e-13)
    _, _, dc = mlp_backward(a, bt, c, do, 1.0)
    np.testing.assert_allclose(np.sum(dc * c), np.sum(do * o), rtol=1e-12)


def test_rows_helper_and_blocks():
    a, bt, c, do = rnd(19, 30, 8), rnd(20, 12, 8), rnd(21, 12, 4), rnd(22, 30, 4)
    o = mlp_forward(a, bt, c, 0.5, block_rows=30, workers=1)
    o2 = mlp_forward(a, bt, c, 0.5, block_rows=4, workers=3)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
    rows = np.array([0, 5, 29])
    np.testing.assert_allclose(mlp_forward_rows(a, bt, c, 0.5, rows), o[rows], rtol=0,
                               atol=1e-14)
    g1 = mlp_backward(a, bt, c, do, 0.5, block_rows=30, workers=1)
    g2 = mlp_backward(a, bt, c, do, 0.5, block_rows=4, workers=3)
    for x, y in zip(g1, g2):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-13)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    from attention_fab_forward_amd.inputs import normal_f32, round_to_bf16
    x = normal_f32(5, (4096,), 3.0)
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 65504.0]
    ref = torch.tensor(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(round_to_bf16(x), ref)
