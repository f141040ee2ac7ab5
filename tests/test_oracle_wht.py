"""Pins for oracle.wht: Sylvester recursion, orthonormality, invariants."""
import numpy as np
import pytest

from oracle import wht


def _sylvester(d):
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_popcount_matrix_is_sylvester(d):
    assert np.array_equal(wht.hadamard_matrix(d), _sylvester(d))


@pytest.mark.parametrize("d", [64, 128])
def test_orthonormal_symmetric_involutory(d):
    h = wht.hadamard_matrix(d)
    assert np.max(np.abs(h @ h.T - np.eye(d))) < 1e-15
    assert np.array_equal(h, h.T)
    assert np.max(np.abs(h @ h - np.eye(d))) < 1e-15


@pytest.mark.parametrize("d", [64, 128])
def test_norm_and_inner_product_preserved(d):
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal((2, 50, d))
    hq, hk = wht.wht_f64(q), wht.wht_f64(k)
    assert np.allclose(np.linalg.norm(hq, axis=1), np.linalg.norm(q, axis=1), rtol=1e-14)
    assert np.allclose(np.sum(hq * hk, axis=1), np.sum(q * k, axis=1), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
def test_butterflies_exact_on_integers(d):
    """Small integers keep every butterfly exact in fp32, so the staged fp32
    transform must equal sqrt(D) * H x exactly."""
    rng = np.random.default_rng(7)
    x = rng.integers(-1000, 1000, size=(40, d)).astype(np.float32)
    ours = wht.fwht_f32_unnormalized(x).astype(np.float64)
    ref = x.astype(np.float64) @ (wht.hadamard_matrix(d) * np.sqrt(d)).T
    assert np.array_equal(ours, np.rint(ref))


@pytest.mark.parametrize("d", [64, 128])
def test_butterflies_fp32_close_to_fp64(d):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((200, d)) * 3).astype(np.float32)
    ours = wht.fwht_f32_unnormalized(x).astype(np.float64) / np.sqrt(d)
    ref = wht.wht_f64(x)
    assert np.max(np.abs(ours - ref)) < 1e-5 * np.max(np.abs(ref))


def test_rsqrt_constant():
    assert wht.rsqrt_dim_f32(64) == np.float32(0.125)
    assert wht.rsqrt_dim_f32(128).view(np.uint32) == np.uint32(0x3DB504F3)
