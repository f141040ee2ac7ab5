"""Pins for oracle.mxfp4: group exponents, element bounds, query cast."""
import numpy as np
import torch

from oracle import fpformats as fp
from oracle import mxfp4, wht
import workloads


def test_value_path_has_no_rotation_and_is_bounded():
    rng = np.random.default_rng(30)
    v = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal((500, 128)).astype(np.float32)))
    codes, x = mxfp4.mx_encode(v)
    vh = mxfp4.mx_decode(codes, x)
    g = v.reshape(500, 4, 32).astype(np.float64)
    amax = np.abs(g).max(-1)
    step = np.exp2(x.astype(np.float64))
    # amax / 2^X lies in [4, 8): values up to 6*2^X have error <= half a grid step (<= 2^X),
    # larger ones are clipped to 6*2^X
    assert np.all((amax / step >= 4) & (amax / step < 8))
    err = np.abs(g - vh.reshape(500, 4, 32))
    clip = np.maximum(np.abs(g) - 6 * step[..., None], 0)
    assert np.all(err <= step[..., None] + clip + 1e-12)


def test_power_of_two_amax_exponent():
    v = np.zeros((1, 128), np.float32)
    v[0, 0] = 8.0           # group 0: amax 8 -> X = 1, 8 / 2 = 4 exactly
    v[0, 40] = -0.5         # group 1: X = -3, -0.5 / 2^-3 = -4
    codes, x = mxfp4.mx_encode(v)
    assert list(x[0]) == [1, -3, -127, -127]
    assert codes[0, 0] == 6 and codes[0, 40] == 14
    assert np.all(mxfp4.mx_decode(codes, x)[0] == v[0])


def test_key_path_rotates_first():
    rng = np.random.default_rng(31)
    k = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal((50, 128)).astype(np.float32)))
    enc = mxfp4.encode_rows(k, k)
    c2, x2 = mxfp4.mx_encode(mxfp4.rotate_f32(k))
    nz = mxfp4.rotate_f32(k) != 0
    assert np.array_equal(enc["kcode"][nz], c2[nz]) and np.array_equal(enc["kexp"], x2)
    y = mxfp4.mx_decode(enc["kcode"], enc["kexp"])
    assert np.max(np.abs(y - wht.wht_f64(k))) < 0.5 * np.max(np.abs(wht.wht_f64(k)))


def test_query_cast_matches_torch_fp8():
    rng = np.random.default_rng(32)
    q = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal((64, 128)).astype(np.float32)))
    ours = mxfp4.query_fp8(q)
    ref = torch.from_numpy(mxfp4.rotate_f32(q)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_zero_signs():
    """A rotated key element that is exactly zero is stored as +0 (code 0);
    values keep the sign of their zeros (OCP: -0 -> code 8)."""
    k = np.full((1, 128), -0.0, np.float32)     # butterflies give -0 and +0 here
    y = mxfp4.rotate_f32(k)
    assert np.any(np.signbit(y)) and np.all(y == 0)
    enc = mxfp4.encode_rows(k, k)
    assert np.all(enc["kcode"] == 0) and np.all(enc["kexp"] == -127)
    assert np.all(enc["vcode"] == 8) and np.all(enc["vexp"] == -127)
    # exact cancellation: k = e0 + e1 rotates to 2/sqrt(D) on even channels, 0 on odd
    k = np.zeros((1, 128), np.float32)
    k[0, :2] = 1.0
    enc = mxfp4.encode_rows(k, np.zeros_like(k))
    y = mxfp4.mx_decode(enc["kcode"], enc["kexp"])[0]
    assert np.all(enc["kcode"][0, 1::2] == 0) and np.all(y[1::2] == 0) and np.all(y[0::2] > 0)
