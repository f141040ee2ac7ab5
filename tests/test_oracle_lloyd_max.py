"""Pins for oracle.lloyd_max: independent quadrature, Monte Carlo, Max (1960)."""
import json
import math
import os

import numpy as np
from scipy import integrate

from oracle import lloyd_max as lm

HERE = os.path.dirname(__file__)


def _levels():
    return lm.lloyd_max_gaussian()


def test_symmetric_and_ascending():
    c = _levels()
    assert np.all(np.diff(c) > 0)
    assert np.max(np.abs(c + c[::-1])) < 1e-14


def test_fixed_point_residual():
    c = _levels()
    assert max(abs(a - b) for a, b in zip(c, lm.centroid_update(list(c)))) < 1e-14


def test_conditional_means_by_quadrature():
    """Each level is the mean of N(0,1) on its cell, by numerical integration
    (independent of the closed form used in the iteration)."""
    c = _levels()
    t = [-np.inf] + list((c[:-1] + c[1:]) / 2) + [np.inf]
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    for i in range(16):
        mass = integrate.quad(pdf, t[i], t[i + 1], epsabs=1e-14, epsrel=1e-13)[0]
        mom = integrate.quad(lambda x: x * pdf(x), t[i], t[i + 1], epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(mom / mass - c[i]) < 1e-9


def test_mse_closed_form_quadrature_and_monte_carlo():
    c = _levels()
    mse = lm.gaussian_mse(c)
    t = [-np.inf] + list((c[:-1] + c[1:]) / 2) + [np.inf]
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    quad = sum(integrate.quad(lambda x, ci=ci: (x - ci) ** 2 * pdf(x), t[i], t[i + 1], epsabs=1e-14)[0]
               for i, ci in enumerate(c))
    assert abs(mse - quad) < 1e-10
    assert abs(mse - 0.0095010) < 5e-7
    x = np.random.default_rng(5).standard_normal(4_000_000)
    idx = np.searchsorted((c[:-1] + c[1:]) / 2, x)
    mc = np.mean((x - c[idx]) ** 2)
    assert abs(mc / mse - 1) < 0.01


def test_published_table():
    g = json.load(open(os.path.join(HERE, "golden", "lloyd_max_gaussian16.json")))
    c = _levels()
    pos = c[8:]
    for ours, printed in zip(pos, g["levels_positive"]):
        assert abs(ours - printed) <= 6e-4, (ours, printed)


def test_default_table_is_one_fp16_rounding():
    t = lm.default_key_table_f16()
    assert t.dtype == np.float16 and len(t) == 16
    c = _levels()
    for ci, ti in zip(c, t.astype(np.float64)):
        # nearest fp16 to ci
        cand = np.array([np.float16(ci), np.nextafter(np.float16(ci), np.float16(np.inf)),
                         np.nextafter(np.float16(ci), np.float16(-np.inf))]).astype(np.float64)
        assert abs(ti - ci) == np.min(np.abs(cand - ci))
    assert abs(lm.gaussian_mse(t.astype(np.float64)) - 0.0095010) < 5e-7
