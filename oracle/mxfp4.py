"""MX-FP4 stretch codecs: FP4 (e2m1) keys and values with UE8M0 group
exponents, FP8 (e4m3) queries.

Test infrastructure only (see ``oracle/__init__``).

[UQ] "方法怎麼做，白話講": UltraQuant replaces the codebook path with a
micro-scaled FP4 representation - FP8 queries, FP4 KV tensors, UE8M0 group
scales - so that dequantization is absorbed into CDNA4's scaled MFMA instead
of a software table lookup; keys are still WHT-rotated (Ultra-TQ keeps the
rotation).  The pages name the formats only.  Readings (OCP MX v1.0 for the
conversions):

* groups of 32 consecutive channels of one (token, kv-head), for keys (after
  rotation) and values (no rotation);
* X = floor(log2(amax)) - 2 clamped to [-127, 127] (amax = 0 -> -127), stored
  as the byte X + 127; element code = e2m1_RNE(x / 2^X), saturating at +-6;
* the rotated key is y = fp32(x * fp32(1/sqrt(D))) with x the fp32 butterflies
  of ``wht.fwht_f32_unnormalized``; a rotated key element that is exactly
  zero is stored as +0 (in exact arithmetic the rotation yields an unsigned
  zero; the sign fp32 gives it depends only on the order of the butterflies'
  operations, not on the data).  Values keep the sign of their zeros;
* the query is rotated the same way and cast to e4m3 (RNE, saturating, unit
  scale); the softmax scale is applied to the fp32 logits.

Every step is exact given the fp32 rotation, so codes compare bit for bit.
Pinned by tests/test_oracle_mxfp4.py (exhaustive e2m1 / e4m3 tables, UE8M0
powers of two, round trips, the value path that has no rotation).
"""
import numpy as np

from . import fpformats as fp
from . import wht

GROUP = 32


def rotate_f32(x):
    """y = fp32(x_butterflies * fp32(1/sqrt(D))) over the last axis."""
    x = np.asarray(x, dtype=np.float32)
    return (wht.fwht_f32_unnormalized(x) * wht.rsqrt_dim_f32(x.shape[-1])).astype(np.float32)


def mx_encode(x):
    """Group-encode [..., D] fp32 values: (e2m1 codes [..., D], X [..., D/32])."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (d // GROUP, GROUP))
    amax = np.abs(g).max(axis=-1)
    xexp = fp.ue8m0_exponent(amax)
    scaled = g.astype(np.float64) * np.exp2(-xexp.astype(np.float64))[..., None]
    codes = fp.e2m1_encode(scaled)
    return codes.reshape(x.shape), xexp


def mx_decode(codes, xexp):
    codes = np.asarray(codes)
    d = codes.shape[-1]
    v = fp.e2m1_decode(codes).reshape(codes.shape[:-1] + (d // GROUP, GROUP))
    return (v * np.exp2(np.asarray(xexp, dtype=np.float64))[..., None]).reshape(codes.shape)


def encode_rows(k, v):
    """FP4-encode key rows (rotated first; zeros as +0) and value rows (not
    rotated)."""
    kc, kx = mx_encode(rotate_f32(k) + np.float32(0.0))
    vc, vx = mx_encode(np.asarray(v, dtype=np.float32))
    return {"kcode": kc, "kexp": kx, "vcode": vc, "vexp": vx}


def query_fp8(q):
    """q -> rotated fp32 -> e4m3 codes (unit scale)."""
    return fp.e4m3_encode(rotate_f32(q))
