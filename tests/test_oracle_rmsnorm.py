"""Pins of the fp64 RMSNorm oracle against things other than itself (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle


def test_torch_rms_norm_float64():
    rng = np.random.default_rng(5)
    for rows, hidden, eps in ((7, 64, 1e-6), (3, 4096, 1e-5), (1, 24, 0.1)):
        x = rng.standard_normal((rows, hidden))
        w = rng.standard_normal(hidden)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (hidden,), torch.from_numpy(w), eps)
        np.testing.assert_allclose(oracle.rmsnorm(x, w, eps), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_pure_python_loops():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 10))
    w = rng.standard_normal(10)
    eps = 0.25
    got = oracle.rmsnorm(x, w, eps)
    for r in range(3):
        ms = sum(float(v) * float(v) for v in x[r]) / 10
        for i in range(10):
            assert abs(got[r, i] - float(x[r, i]) / math.sqrt(ms + eps) * float(w[i])) < 1e-14


def test_constant_rows_closed_form():
    w = np.array([1.0, -2.0, 0.5, 3.0])
    for c, eps in ((2.0, 0.0), (-3.0, 0.0), (0.5, 0.75)):
        x = np.full((1, 4), c)
        exp = c / math.sqrt(c * c + eps) * w
        np.testing.assert_allclose(oracle.rmsnorm(x, w, eps)[0], exp, rtol=0, atol=1e-15)


def test_scale_invariance_and_mean_square():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 128))
    w = rng.uniform(0.5, 2.0, 128)
    np.testing.assert_allclose(oracle.rmsnorm(3.5 * x, w, 0.0), oracle.rmsnorm(x, w, 0.0), rtol=1e-13)
    eps = 0.3
    y = oracle.rmsnorm(x, w, eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean((y / w) ** 2, axis=1), ms / (ms + eps), rtol=1e-13)


@pytest.mark.parametrize("slip", ["sum_not_mean", "no_eps", "no_weight", "weight_on_rows"])
def test_pins_catch_planted_mistakes(slip):
    """Copies of the definition with a plausible slip fail the torch pin."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 32))
    w = rng.standard_normal(32)
    eps = 0.5
    if slip == "sum_not_mean":
        bad = x / np.sqrt(np.sum(x * x, axis=1, keepdims=True) + eps) * w
    elif slip == "no_eps":
        bad = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True)) * w
    elif slip == "no_weight":
        bad = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    else:
        bad = x / np.sqrt(np.mean(x * x, axis=0, keepdims=True) + eps) * w
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (32,), torch.from_numpy(w), eps).numpy()
    assert not np.allclose(bad, ref, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(oracle.rmsnorm(x, w, eps), ref, rtol=1e-13, atol=1e-13)
