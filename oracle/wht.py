"""The orthonormal Walsh-Hadamard rotation.

Test infrastructure only (see ``oracle/__init__``).

[TQ-AMD] section 4 ("Walsh-Hadamard 比隨機 rotation 更實用") and [UQ]
"方法怎麼做，白話講": keys are rotated with a Walsh-Hadamard transform before
quantization (it spreads outlier channels and is easy to put in a kernel);
values are not rotated ([TQ-AMD] section 2: V uses plain uniform quantization).
The rotation is orthonormal, so rotating the query by the same matrix leaves
every query-key product unchanged.

Reading (the pages give neither): natural (Sylvester) ordering,
    H_D[i, j] = (-1)^popcount(i & j) / sqrt(D),
with no random sign flips (the pages contrast WHT *with* random rotation).

Two forms:
* ``hadamard_matrix`` / ``wht_f64`` - the plain definition, fp64.
* ``fwht_f32_unnormalized`` - the same transform as log2(D) butterfly stages
  in fp32, in the fixed order h = 1, 2, 4, ..., D/2, each stage replacing
  (x[i], x[i+h]) for (i & h) == 0 by (x[i] + x[i+h], x[i] - x[i+h]), each sum
  rounded once to fp32.  This is the precision in which the kernels take the
  code decisions, so the oracle takes them the same way (see ``tq4``).  The
  1/sqrt(D) normalization is applied by the caller where stated.

Pinned by tests/test_oracle_wht.py: the popcount matrix equals the recursive
Sylvester construction, H H^T = I, H = H^T, norm and inner-product
preservation, butterflies == matrix product (fp64), fp32 butterflies within
rounding of fp64.
"""
import math

import numpy as np


def hadamard_matrix(d):
    """H_d[i, j] = (-1)^popcount(i & j) / sqrt(d), fp64."""
    if d <= 0 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0) / math.sqrt(d)


def wht_f64(x):
    """Rotate the last axis of ``x`` by H_D in fp64 (explicit matrix product)."""
    x = np.asarray(x, dtype=np.float64)
    h = hadamard_matrix(x.shape[-1])
    return x @ h.T


def fwht_f32_unnormalized(x):
    """Unnormalized Walsh-Hadamard butterflies over the last axis, in fp32.

    Stage order h = 1, 2, ..., D/2; pairs (i, i+h) with (i & h) == 0 become
    (a + b, a - b), each rounded to fp32.  Returns sqrt(D) * H_D x up to fp32
    rounding.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < d:
        idx = np.arange(d)
        lo = idx[(idx & h) == 0]
        hi = lo + h
        a = y[..., lo].copy()
        b = y[..., hi].copy()
        y[..., lo] = a + b          # fp32 + fp32 -> fp32 (one rounding)
        y[..., hi] = a - b
        h *= 2
    return y


def rsqrt_dim_f32(d):
    """fp32 value of 1/sqrt(d), correctly rounded (exact for d = 64)."""
    return np.float32(1.0 / math.sqrt(d))
