"""TQ4/4 codecs: 4-bit keys (rotation + 16-entry table) and 4-bit values
(per-group asymmetric uniform).

Test infrastructure only (see ``oracle/__init__``).

Sources on the pages:
* [TQ-AMD] section 2 ("TQ4/4 是最穩的預設值"): TQ4/4 means 4-bit K and 4-bit V;
  keys are more sensitive, so K uses rotation plus LUT quantization while V uses
  standard uniform quantization.
* [TQ-AMD] section 4 and [UQ] "方法怎麼做，白話講": the rotation is a
  Walsh-Hadamard transform; the key table has 16 entries and starts from the
  Lloyd-Max centroids.
* [TQ-AMD] section 5: no QJL residual at 4 bits.

Readings where the pages are silent (each listed in the design notes):
* Key scale: one per (token, kv-head), the RMS of the key,
  s = fp16_RNE(sqrt(sum_i k_i^2 / D)), evaluated exactly (the bf16 squares sum
  exactly in fp64 whenever a row's squares span less than 2^37, i.e. for any
  realistic row), saturated to 65504.  RMS makes y/s ~ N(0,1) for the N(0,1)
  table.
* Key code: the nearest table entry to y_i / s, ties to the lower index, with
  the decision taken in fp32 in this fixed order:
      x   = unnormalized fp32 butterflies of k (``wht.fwht_f32_unnormalized``)
      w   = fp32( fp32(1/s) * fp32(1/sqrt(D)) )          (s > 0)
      u_i = fp32( x_i * w )                              (u = 0 when s = 0)
      t_j = fp32( (c_j + c_{j+1}) * 0.5 ),  j = 0..14    (c = fp16 table)
      code_i = #{ j : u_i > t_j }
  ``key_codes_exact`` is the exact fp64 nearest-entry rule; the two agree except
  where the fp64 distance gap is below 1e-5 (flagged near-ties).
* Key dequantization: k_hat_rot = c[code] * s, exact in fp32; keys stay in the
  rotated domain and the query is rotated instead.
* Value groups: 32 consecutive channels of one (token, kv-head); per group
      mn = min, mx = max (exact),  sc = fp16_sat(fp32(fp32(mx - mn) / 15)),
      mn16 = fp16_sat(mn),
      code = clamp(RNE(fp32(fp32(v - mn16) * fp32(1/sc))), 0, 15)   (sc > 0)
      code = 0                                                      (sc = 0)
      v_hat = fp32(code * sc + mn16)      (one rounding; code*sc is exact)
  ``value_codes_exact`` is the exact rule RNE((v - mn16)/sc) in fp64 with its
  near-tie flags.

TQ4/2 ([TQ-AMD] section 2 names 2-bit variants as feasible but of little
pay-off): keys as above; values take the same per-group rule with 2-bit codes,
sc = fp16_sat(fp32(fp32(mx - mn) / 3)) and codes clamped to 0 .. 3 (the
plainest reading: the 4-bit rule with 2^2 - 1 levels).

Pinned by tests/test_oracle_tq4.py: centroid round trip (encode(c_j * s) = j),
agreement with the exact rules away from flagged near-ties, hand-computed
vectors and groups (tests/golden/), error bounds, idempotence, zero / constant
/ saturated special cases.
"""
import numpy as np

from . import fpformats as fp
from . import wht

GROUP = 32


# ---------------------------------------------------------------------------
# keys
# ---------------------------------------------------------------------------

def key_scale(k):
    """Per-row key scale s = fp16_RNE(RMS(k)) for fp32 keys (bf16 values)."""
    k = np.asarray(k, dtype=np.float32).astype(np.float64)
    ms = np.sum(k * k, axis=-1) / k.shape[-1]          # exact sum of bf16 squares
    return fp.f16_rne_sqrt_exact(ms)


def key_midpoints_f32(table_f16):
    """t_j = fp32((c_j + c_{j+1}) * 0.5) for the fp16 table (15 values)."""
    c = np.asarray(table_f16, dtype=np.float16).astype(np.float32)
    return ((c[:-1] + c[1:]) * np.float32(0.5)).astype(np.float32)


def key_unit_coords_f32(k, s):
    """u = fp32(x * w): rotated key in units of its scale, as the decision
    precision defines it (see the module docstring)."""
    k = np.asarray(k, dtype=np.float32)
    d = k.shape[-1]
    x = wht.fwht_f32_unnormalized(k)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv_s = np.where(s32 > 0, np.float32(1.0) / np.where(s32 > 0, s32, np.float32(1.0)), np.float32(0.0))
    w = (inv_s.astype(np.float32) * wht.rsqrt_dim_f32(d)).astype(np.float32)
    u = (x * w[..., None]).astype(np.float32)
    return np.where((s32 > 0)[..., None], u, np.float32(0.0)).astype(np.float32)


def key_codes_from_units(u, table_f16):
    """Code of each fp32 unit coordinate: #{ j : u > t_j } (nearest table
    entry, ties to the lower index, in fp32)."""
    t = key_midpoints_f32(table_f16)
    return np.sum(np.asarray(u, dtype=np.float32)[..., None] > t, axis=-1).astype(np.uint8)


def key_codes(k, s, table_f16):
    """4-bit key codes of rows k [..., D] with scales s [...] (fp32 rule)."""
    return key_codes_from_units(key_unit_coords_f32(k, s), table_f16)


def key_codes_exact(k, s, table_f16, tie_tol=1e-5):
    """The exact rule: argmin_j |y_i/s - c_j| in fp64 (ties to the lower index),
    y = H_D k exactly.  Returns (codes, near_tie) where near_tie marks
    elements whose best and second-best distances differ by < ``tie_tol``."""
    y = wht.wht_f64(np.asarray(k, dtype=np.float32))
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)
    u = np.where((s64 > 0)[..., None], y / np.where(s64 > 0, s64, 1.0)[..., None], 0.0)
    c = np.asarray(table_f16, dtype=np.float16).astype(np.float64)
    dist = np.abs(u[..., None] - c)
    codes = np.argmin(dist, axis=-1)                # first minimum = lower index
    ds = np.sort(dist, axis=-1)
    near = (ds[..., 1] - ds[..., 0]) < tie_tol
    return codes.astype(np.uint8), near


def key_dequant_rot(codes, s, table_f16):
    """k_hat in the rotated domain: c[code] * s (exact in fp32)."""
    c = np.asarray(table_f16, dtype=np.float16).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)
    return (c[np.asarray(codes, dtype=np.int64)] * s32[..., None]).astype(np.float32)


# ---------------------------------------------------------------------------
# values
# ---------------------------------------------------------------------------

def _groups(v):
    v = np.asarray(v, dtype=np.float32)
    d = v.shape[-1]
    if d % GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    return v.reshape(v.shape[:-1] + (d // GROUP, GROUP))


def value_scale_min(v, levels=15):
    """Per-32-channel group (sc, mn16) as fp16 (see module docstring);
    ``levels`` = 2^bits - 1 (15 for 4-bit values, 3 for 2-bit)."""
    g = _groups(v)
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    rng = (mx - mn).astype(np.float32)
    sc = fp.f32_to_f16_sat((rng / np.float32(levels)).astype(np.float32))
    mn16 = fp.f32_to_f16_sat(mn)
    return sc, mn16


def value_codes(v, sc, mn16, levels=15):
    """Value codes (0 .. levels) in the fp32 decision precision."""
    g = _groups(v)
    sc32 = np.asarray(sc, dtype=np.float16).astype(np.float32)
    mn32 = np.asarray(mn16, dtype=np.float16).astype(np.float32)
    pos = sc32 > 0
    inv = np.where(pos, np.float32(1.0) / np.where(pos, sc32, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    d = (g - mn32[..., None]).astype(np.float32)
    q = (d * inv[..., None]).astype(np.float32)
    code = np.clip(np.rint(q), 0, levels)
    code = np.where(pos[..., None], code, 0).astype(np.uint8)
    return code.reshape(np.asarray(v).shape)


def value_encode(v, levels=15):
    sc, mn16 = value_scale_min(v, levels)
    return value_codes(v, sc, mn16, levels), sc, mn16


def value_codes_exact(v, sc, mn16, tie_tol=1e-5, levels=15):
    """Exact rule clamp(RNE((v - mn16)/sc), 0, levels) in fp64, with near-tie
    flags where (v - mn16)/sc lies within ``tie_tol`` of a half-integer."""
    g = _groups(v).astype(np.float64)
    sc64 = np.asarray(sc, dtype=np.float16).astype(np.float64)
    mn64 = np.asarray(mn16, dtype=np.float16).astype(np.float64)
    pos = sc64 > 0
    q = (g - mn64[..., None]) / np.where(pos, sc64, 1.0)[..., None]
    code = np.where(pos[..., None], np.clip(np.rint(q), 0, levels), 0)
    frac = np.abs(q - np.floor(q) - 0.5)
    near = pos[..., None] & (frac < tie_tol) & (q > -0.5) & (q < levels + 0.5)
    shape = np.asarray(v).shape
    return code.astype(np.uint8).reshape(shape), near.reshape(shape)


def value_dequant(codes, sc, mn16):
    """v_hat = fp32(code * sc + mn16), one rounding."""
    c = _groups(np.asarray(codes, dtype=np.float32)).astype(np.float64)
    sc64 = np.asarray(sc, dtype=np.float16).astype(np.float64)
    mn64 = np.asarray(mn16, dtype=np.float16).astype(np.float64)
    out = (c * sc64[..., None] + mn64[..., None]).astype(np.float32)
    return out.reshape(np.asarray(codes).shape)


# ---------------------------------------------------------------------------
# one (token, kv-head) row, both halves
# ---------------------------------------------------------------------------

def encode_rows(k, v, table_f16, vlevels=15):
    """Encode key and value rows [..., D] (fp32 holding bf16 values);
    ``vlevels`` 15 (TQ4/4) or 3 (TQ4/2: 2-bit values).

    Returns dict(kcode, kscale, vcode, vscale, vmin)."""
    s = key_scale(k)
    kc = key_codes(k, s, table_f16)
    vc, sc, mn = value_encode(v, vlevels)
    return {"kcode": kc, "kscale": s, "vcode": vc, "vscale": sc, "vmin": mn}
