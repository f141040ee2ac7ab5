"""Pins of the calibrated-table oracle (oracle/calibrate.py) to facts outside
it: the Lloyd-Max quantizer of N(0,1) (Max 1960) and the uniform quantizer as
limits of the fit, the two Lloyd conditions checked by brute force, the
monotone distortion, exact scale equivariance, a hand-worked cluster case, the
MSE against an explicit inverse rotation and the Gaussian Lloyd-Max MSE, and
hand-worked layer choices."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import ndtri

import workloads
from oracle import calibrate, lloyd_max, tq4, wht

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def test_gaussian_quantile_sample_converges_to_max_table():
    # A Gaussian quantile sample is a discretized N(0,1); its Lloyd fixed point
    # lies within the discretization of the Lloyd-Max table (Max 1960, Table I).
    g = json.load(open(os.path.join(GOLDEN, "lloyd_max_gaussian16.json")))
    pos = np.array(g["levels_positive"], dtype=np.float64)
    ref = np.concatenate([-pos[::-1], pos])
    n = 100000
    u = ndtri((np.arange(n) + 0.5) / n)
    init = lloyd_max.default_key_table_f16().astype(np.float64) * 1.05
    levels, updates = calibrate.lloyd_fit(u, init, max_iters=2000)
    assert updates < 2000
    assert np.max(np.abs(levels - ref)) < 2.5e-3


def test_uniform_sample_converges_to_uniform_quantizer():
    n = 100000
    u = (np.arange(n) + 0.5) / n * 2.0 - 1.0
    init = np.linspace(-0.9, 0.9, 16) ** 3
    levels, updates = calibrate.lloyd_fit(u, init, max_iters=5000)
    assert updates < 5000
    assert np.max(np.abs(levels - ((2 * np.arange(16) + 1) / 16.0 - 1.0))) < 1e-3


def test_fixed_point_meets_both_lloyd_conditions():
    g = np.random.default_rng(5)
    u = g.standard_t(4, size=6000) * 0.8
    init = lloyd_max.default_key_table_f16().astype(np.float64)
    levels, updates = calibrate.lloyd_fit(u, init, max_iters=100000)
    assert updates < 100000
    # nearest-neighbour condition, by brute-force distances (first minimum)
    near = np.argmin(np.abs(u[:, None] - levels[None, :]), axis=1)
    # centroid condition, by an exactly rounded sum
    for j in range(16):
        members = u[near == j]
        assert members.size > 0
        assert levels[j] == pytest.approx(math.fsum(members) / members.size, rel=1e-14, abs=1e-15)
    assert np.all(np.diff(levels) > 0)


def test_distortion_never_increases():
    g = np.random.default_rng(6)
    u = np.concatenate([g.normal(-1.2, 0.3, 3000), g.normal(1.0, 0.5, 3000), g.laplace(0, 2, 500)])
    hist = []
    calibrate.lloyd_fit(u, lloyd_max.default_key_table_f16().astype(np.float64), max_iters=60, history=hist)
    d = np.array(hist)
    assert len(d) >= 10
    assert np.all(d[1:] <= d[:-1] * (1 + 1e-12))
    assert d[-1] < d[0]


def test_power_of_two_scale_equivariance():
    g = np.random.default_rng(7)
    u = g.standard_t(5, size=4000)
    init = lloyd_max.default_key_table_f16().astype(np.float64)
    a, na = calibrate.lloyd_fit(u, init, max_iters=40)
    b, nb = calibrate.lloyd_fit(4.0 * u, 4.0 * init, max_iters=40)
    assert na == nb
    assert np.array_equal(b, 4.0 * a)


def test_hand_worked_clusters_and_empty_cell():
    # 16 clusters {m - 1/4, m, m + 1/4} with m = j - 7.5; starting 0.1 above
    # each mean, every cluster is its own cell, so one update lands on the
    # exact means and the next changes nothing.
    m = np.arange(16) - 7.5
    u = np.concatenate([m - 0.25, m, m + 0.25])
    levels, updates = calibrate.lloyd_fit(u, m + 0.1, max_iters=10)
    assert updates == 1
    assert np.array_equal(levels, m)
    # without cluster 5, cell 5 stays empty and keeps its starting value
    u5 = u[np.abs(np.concatenate([m, m, m]) - m[5]) > 1e-9]
    levels, updates = calibrate.lloyd_fit(u5, m + 0.1, max_iters=10)
    assert updates == 1
    expect = m.copy()
    expect[5] = m[5] + 0.1
    assert np.array_equal(levels, expect)


def test_max_iters_zero_returns_the_start():
    u = np.linspace(-3, 3, 101)
    init = lloyd_max.default_key_table_f16().astype(np.float64)
    levels, updates = calibrate.lloyd_fit(u, init, max_iters=0)
    assert updates == 0 and np.array_equal(levels, init)


def test_fit_samples_leave_out_zero_rows():
    g = np.random.default_rng(8)
    k = _bf16(g.normal(size=(6, 64)))
    kz = np.concatenate([k[:3], np.zeros((2, 64), np.float32), k[3:]])
    assert np.array_equal(calibrate.fit_samples(k), calibrate.fit_samples(kz))
    assert calibrate.fit_samples(k).size == 6 * 64


@pytest.mark.parametrize("d", [64, 128])
def test_key_mse_equals_error_in_key_coordinates(d):
    g = np.random.default_rng(9 + d)
    k = _bf16(g.standard_t(4, size=(40, d)) + g.normal(0, 0.5, size=(1, d)))
    k[3] = 0.0
    table = lloyd_max.default_key_table_f16()
    s = tq4.key_scale(k)
    codes = tq4.key_codes(k, s, table)
    c = table.astype(np.float64)
    # dequantize, rotate back with the explicit matrix, compare in k's coordinates
    khat = (c[codes.astype(np.int64)] * s.astype(np.float64)[:, None]) @ wht.hadamard_matrix(d)
    direct = np.mean((khat - k.astype(np.float64)) ** 2)
    assert calibrate.key_mse(k, table) == pytest.approx(direct, rel=1e-12)


def test_key_mse_of_gaussian_keys_is_lloyd_max_mse():
    # N(0,1) keys have unit RMS; after the rotation the unit coordinates are
    # close to N(0,1), whose Lloyd-Max MSE is 0.009501 (closed form).
    g = np.random.default_rng(10)
    k = _bf16(g.standard_normal(size=(3000, 128)))
    mse = calibrate.key_mse(k, lloyd_max.default_key_table_f16())
    assert mse == pytest.approx(0.009501, rel=0.04)


def test_fitted_table_lowers_mse_on_two_valued_rows():
    # a single dominant channel makes every rotated entry +-a: the N(0,1) table
    # fits that badly and the fitted one much better
    g = np.random.default_rng(11)
    k = g.standard_normal(size=(160, 128)).astype(np.float32)
    k[:, 17] *= 40.0
    k = _bf16(k)
    init = lloyd_max.default_key_table_f16()
    table, levels, updates = calibrate.fit_table(k, init, max_iters=100)
    assert updates > 0
    assert np.all(np.diff(table.astype(np.float64)) > 0)
    assert calibrate.key_mse(k, table) < 0.75 * calibrate.key_mse(k, init)


def test_layer_choice_by_hand():
    assert calibrate.select_layers([]).tolist() == []
    assert calibrate.select_layers([0.3]).tolist() == [True]
    m10 = [0.1, 0.5, 0.2, 0.05, 0.3, 0.25, 0.15, 0.12, 0.11, 0.4]
    assert calibrate.select_layers(m10).nonzero()[0].tolist() == [1]
    # 32 layers: ranks 0..3 (4 < 3.2 is false, 3 < 3.2 true)
    m32 = np.arange(32, dtype=np.float64)[::-1] * 0.01
    assert calibrate.select_layers(m32).nonzero()[0].tolist() == [0, 1, 2, 3]
    # 30 layers: exactly 3, no floating-point slip to 4
    m30 = np.linspace(1, 2, 30)
    assert calibrate.select_layers(m30).nonzero()[0].tolist() == [27, 28, 29]
    # equal MSEs: lower index first
    assert calibrate.select_layers([1.0] * 20).nonzero()[0].tolist() == [0, 1]
    assert not calibrate.select_layers(m10, percent=0).any()
    assert calibrate.select_layers(m10, percent=100).all()
