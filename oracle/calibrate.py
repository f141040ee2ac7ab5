"""Calibrated key tables: a Lloyd fit of the 16 table entries on captured keys,
the per-element key-quantization MSE of a layer, and the choice of the layers
that get a fitted table.

Test infrastructure only (see ``oracle/__init__``).

Source: [UQ] "方法怎麼做，白話講". Instead of keeping only the theoretical
Lloyd-Max centroids, the 16-entry key table is refit on captured activations.
The calibration needs about 20 vectors per rotated layer from one forward
pass, and the fitted table is used only on the tenth of the layers with the
highest per-element key-quantization MSE.  [UQ] "它實際證明了什麼" reports the
effect as a per-element K MSE drop of about 10% on real activations (not
reproducible here: parity unpinned for that figure).

Readings where the page is silent (each listed in the design notes):
* Samples.  The fit runs on the values the key coder actually quantizes: the
  unit coordinates u = y / s of every element of every calibration key row of
  the layer (``tq4.key_unit_coords_f32``: the fp32 decision precision), all
  kv-heads pooled, because a cache, and so a table, is per layer.  Rows whose
  scale is 0 (all-zero keys) decode to 0 whatever the table and are left out
  of the fit.
* Algorithm.  Lloyd's iteration for a scalar quantizer (S. P. Lloyd, "Least
  squares quantization in PCM", 1957/1982), in fp64, started from the table in
  use (normally the N(0,1) Lloyd-Max table rounded to fp16):
      assignment:  cell(u) = #{ j : u > (c_j + c_{j+1}) / 2 }   (ties to the
                   lower entry: nearest entry for ascending c)
      update:      c_j = mean of the samples in cell j (a zero mean is +0);
                   an empty cell keeps c_j
  and stop when an update leaves every entry unchanged (a fixed point) or after
  ``max_iters`` updates.  The fitted table is each entry rounded once to fp16.
* MSE.  Per-element mean of the squared key error of the cache as the coder
  writes it: codes by the fp32 rule with the fp16 table, dequantized key
  c16[code] * s16, compared with the exact rotated key y = H_D k in fp64.  H_D
  is orthonormal, so this equals the mean squared error in the key's own
  coordinates.  Every calibration element counts (all-zero rows add 0).
* Choice of layers.  Layers are ranked by that MSE under the table in use,
  largest first (equal MSE: lower layer index first); the layer at rank r
  (0-based) is chosen when r < L / 10 (exactly: 100 r < 10 L), so 32 layers
  give 4 and 10 layers give 1.

Pinned by tests/test_oracle_calibrate.py: convergence to Max's N(0,1) table on a
Gaussian quantile sample and to the uniform quantizer on a uniform one; the two
Lloyd conditions at the fixed point checked by brute-force nearest entries and
plain means; non-increasing distortion; exact power-of-two scale equivariance;
a hand-worked cluster case; the MSE against an explicit inverse rotation in the
key's own coordinates and against the Gaussian Lloyd-Max MSE; hand-worked
layer choices.
"""
import numpy as np

from . import tq4
from . import wht

LEVELS = 16


def lloyd_fit(samples, init, max_iters=100, history=None):
    """Lloyd's iteration on 1-D ``samples`` (fp64) from the ascending ``init``
    levels.  Returns (levels fp64 [16], updates performed).  When ``history``
    is a list, the distortion mean((u - c[cell(u)])^2) before each update and
    after the last one is appended to it."""
    u = np.asarray(samples, dtype=np.float64).ravel()
    c = np.array(init, dtype=np.float64)
    updates = 0
    for _ in range(max_iters + 1):
        t = (c[:-1] + c[1:]) * 0.5
        cell = np.sum(u[:, None] > t[None, :], axis=1)
        if history is not None:
            history.append(float(np.mean((u - c[cell]) ** 2)) if u.size else 0.0)
        if updates == max_iters:
            break
        new = c.copy()
        for j in range(LEVELS):
            members = u[cell == j]
            if members.size:
                new[j] = np.sum(members) / members.size + 0.0   # a zero mean is +0
        if np.array_equal(new, c):
            break
        c = new
        updates += 1
    return c, updates


def fit_samples(k_rows):
    """The fit's samples for key rows k [R, D] (bf16 values as fp32): the unit
    coordinates of the rows whose scale is nonzero."""
    k = np.asarray(k_rows, dtype=np.float32)
    s = tq4.key_scale(k)
    u = tq4.key_unit_coords_f32(k, s)
    return u[s.astype(np.float32) > 0].astype(np.float64).ravel()


def fit_table(k_rows, init_table_f16, max_iters=100):
    """Fit one layer's table on its calibration key rows [R, D].  Returns
    (fp16 table [16], fp64 levels [16], updates)."""
    init = np.asarray(init_table_f16, dtype=np.float16).astype(np.float64)
    levels, updates = lloyd_fit(fit_samples(k_rows), init, max_iters)
    return levels.astype(np.float16), levels, updates


def key_mse(k_rows, table_f16):
    """Per-element mean squared error of keys [R, D] coded with ``table_f16``
    (fp32 code rule, fp16 scale), measured against the exact rotation."""
    k = np.asarray(k_rows, dtype=np.float32)
    if k.size == 0:
        return 0.0
    s = tq4.key_scale(k)
    codes = tq4.key_codes(k, s, table_f16)
    c = np.asarray(table_f16, dtype=np.float16).astype(np.float64)
    khat = c[codes.astype(np.int64)] * s.astype(np.float64)[:, None]
    y = wht.wht_f64(k)
    return float(np.mean((khat - y) ** 2))


def select_layers(mse, percent=10):
    """Boolean mask of the layers that get a fitted table: rank r (by MSE,
    largest first, equal values by lower index) is chosen when
    r < percent/100 * L, compared exactly in integers."""
    mse = np.asarray(mse, dtype=np.float64)
    n = mse.size
    order = sorted(range(n), key=lambda i: (-mse[i], i))
    chosen = np.zeros(n, dtype=bool)
    for r, i in enumerate(order):
        if 100 * r < percent * n:
            chosen[i] = True
    return chosen
