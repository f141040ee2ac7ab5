"""The 16-level Lloyd-Max quantizer of the standard normal distribution.

Test infrastructure only (see ``oracle/__init__``).

[UQ] "方法怎麼做，白話講" names the theoretical Lloyd-Max centroids as the
starting point of the 16-entry key table (later refit on captured activations).
Keys are coded after the WHT rotation and division by their RMS scale, so the
coordinates the table sees are close to N(0,1); the default table is therefore
the Lloyd-Max quantizer of N(0,1).

Lloyd's two conditions, iterated to a fixed point in fp64:
  * each threshold is the midpoint of its two neighbouring levels,
        t_i = (c_i + c_{i+1}) / 2;
  * each level is the conditional mean of N(0,1) on its cell (t_{i-1}, t_i),
        c_i = (phi(t_{i-1}) - phi(t_i)) / (Phi(t_i) - Phi(t_{i-1})),
    with phi, Phi the standard normal density and distribution function
    (the closed form of the integral of x*phi(x)).

Pinned by tests/test_oracle_lloyd_max.py: the conditional means checked by
independent numerical quadrature, symmetry, the fixed-point residual, the
mean-squared error against Monte-Carlo sampling, and the published 16-level
Gaussian table (Max, 1960) to its printed 4 digits.
"""
import math

import numpy as np

LEVELS = 16


def _phi(x):
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _Phi(x):
    if x == -math.inf:
        return 0.0
    if x == math.inf:
        return 1.0
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def thresholds(levels):
    """Midpoints between consecutive levels (Lloyd's nearest-neighbour rule)."""
    c = list(levels)
    return [(c[i] + c[i + 1]) / 2.0 for i in range(len(c) - 1)]


def centroid_update(levels):
    """One Lloyd step: the conditional means of N(0,1) on the current cells."""
    t = [-math.inf] + thresholds(levels) + [math.inf]
    out = []
    for i in range(len(levels)):
        a, b = t[i], t[i + 1]
        out.append((_phi(a) - _phi(b)) / (_Phi(b) - _Phi(a)))
    return out


def lloyd_max_gaussian(n=LEVELS, tol=1e-15, max_iter=100000):
    """Fixed point of the Lloyd iteration for N(0,1) with ``n`` levels (fp64).

    Starts from a uniform table on [-3, 3] and iterates until no level moves
    by more than ``tol``.  Returns the ascending levels as a float64 array.
    """
    c = [-3.0 + 6.0 * (i + 0.5) / n for i in range(n)]
    for _ in range(max_iter):
        nc = centroid_update(c)
        moved = max(abs(x - y) for x, y in zip(c, nc))
        c = nc
        if moved <= tol:
            break
    return np.array(c, dtype=np.float64)


def gaussian_mse(levels):
    """Mean-squared error of nearest-level quantization of N(0,1), closed form.

    On a cell (a, b) with level c:  E[(X - c)^2; a < X < b]
      = [Phi(b) - Phi(a)] (1 + c^2) + a phi(a) - b phi(b) - 2c (phi(a) - phi(b)),
    using the integrals of x^2 phi and x phi over the cell.
    """
    t = [-math.inf] + thresholds(levels) + [math.inf]
    total = 0.0
    for i, c in enumerate(levels):
        a, b = t[i], t[i + 1]
        pa = _phi(a)
        pb = _phi(b)
        mass = _Phi(b) - _Phi(a)
        apa = 0.0 if math.isinf(a) else a * pa
        bpb = 0.0 if math.isinf(b) else b * pb
        total += mass * (1.0 + c * c) + apa - bpb - 2.0 * c * (pa - pb)
    return total


def default_key_table_f16():
    """The default 16-entry key table as stored: each level rounded to fp16
    (round to nearest even).  A reading: the pages do not give the storage
    precision; fp16 makes every dequantized key (level x fp16 scale) exact in
    fp32."""
    return lloyd_max_gaussian().astype(np.float16)   # one rounding, fp64 -> fp16
