"""Pins of the fp64 GEMM oracle against things other than itself (CPU only)."""

import numpy as np

import oracle


def test_pure_python_loops():
    rng = np.random.default_rng(9)
    a = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    got = oracle.gemm(a, w)
    for i in range(3):
        for j in range(4):
            assert abs(got[i, j] - sum(float(a[i, k]) * float(w[j, k]) for k in range(5))) < 1e-13


def test_identity_and_one_hot():
    rng = np.random.default_rng(10)
    a = rng.standard_normal((6, 8))
    np.testing.assert_array_equal(oracle.gemm(a, np.eye(8)), a)        # W = I gives A
    w = np.zeros((3, 8)); w[0, 2] = 1.0; w[1, 7] = 2.0; w[2, 0] = -1.0
    np.testing.assert_array_equal(oracle.gemm(a, w), np.stack([a[:, 2], 2 * a[:, 7], -a[:, 0]], 1))


def test_transpose_is_on_w():
    """A transposed operand (A W instead of A W^T) would fail on non-square shapes."""
    a = np.arange(6.0).reshape(2, 3)
    w = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 1.0]])
    np.testing.assert_array_equal(oracle.gemm(a, w), np.array([[0.0, 2.0], [3.0, 5.0]]))


def test_linearity_in_a():
    rng = np.random.default_rng(11)
    a1, a2 = rng.standard_normal((4, 16)), rng.standard_normal((4, 16))
    w = rng.standard_normal((5, 16))
    np.testing.assert_allclose(oracle.gemm(2 * a1 - a2, w), 2 * oracle.gemm(a1, w) - oracle.gemm(a2, w),
                               rtol=1e-12, atol=1e-12)
