"""Pins for the oracle's Sylvester-Hadamard matrix and rotation (CPU only).

[TACO pt-summary, 2.B.1]: the rotation is an orthogonal Hadamard transform that
preserves energy.  Pins: the defining identity H H^T = n I, equality with
scipy.linalg.hadamard (an independent library routine, Sylvester order), and a
butterfly (fast Walsh-Hadamard) evaluation written here as a different algorithm.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024])
def test_hadamard_orthogonality_and_scipy(n):
    H = oracle.hadamard(n)
    assert np.array_equal(H @ H.T, n * np.eye(n))
    assert np.array_equal(H, scipy.linalg.hadamard(n).astype(np.float64))
    Q = H / np.sqrt(n)
    assert np.allclose(Q @ Q, np.eye(n), atol=1e-12)     # symmetric and orthonormal


def test_hadamard_rejects_non_power_of_two():
    for n in (0, 3, 12, 100):
        with pytest.raises(ValueError):
            oracle.hadamard(n)


def butterfly(v):
    """In-place radix-2 Walsh-Hadamard butterflies along the last axis."""
    v = v.copy()
    n = v.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v


@pytest.mark.parametrize("B", [4, 64, 128, 256])
def test_rotation_equals_butterflies_and_preserves_energy(B):
    rng = np.random.default_rng(B)
    xb = rng.standard_normal((16, B))
    alpha = rng.uniform(0.5, 2.0, 16).astype(np.float32)
    y = oracle.hadamard_rotate(xb, alpha)
    ref = alpha.astype(np.float64)[:, None] * butterfly(xb) / np.sqrt(B)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    # Parseval: ||y_k|| = alpha_k ||x_k||
    assert np.allclose(np.linalg.norm(y, axis=1),
                       alpha.astype(np.float64) * np.linalg.norm(xb, axis=1), rtol=1e-13)
    # unit vectors map to the scaled columns of H
    e = np.eye(B)
    assert np.allclose(oracle.hadamard_rotate(e, np.ones(B, np.float32)),
                       oracle.hadamard(B).T / np.sqrt(B), atol=1e-15)
