"""Number formats used by the codecs, written from their definitions.

Test infrastructure only (see ``oracle/__init__``).

* bf16 -> fp32 widening (exact).
* fp32 -> fp16 round-to-nearest-even, plain and saturating.
* the exact fp16 rounding of a square root (used by the key scale).
* OCP FP8 e4m3fn encode/decode (bias 7, max 448, no infinities, RNE,
  saturate to finite) - named on [UQ] "方法怎麼做，白話講" (FP8 queries); the
  bit format is the OCP 8-bit floating point specification.
* OCP FP4 e2m1 encode/decode (values 0, .5, 1, 1.5, 2, 3, 4, 6 with a sign,
  RNE with ties to the even code, saturate at +-6) and the UE8M0 exponent
  scale - named on [UQ] "方法怎麼做，白話講" (FP4 KV tensors, UE8M0 group
  scales); the bit formats are the OCP Microscaling (MX) v1.0 specification.

Pinned by tests/test_oracle_formats.py: torch's own fp16 / float8_e4m3fn
conversions on dense samples, exhaustive decode tables, and hand tie cases.
"""
import math

import numpy as np

F16_MAX = 65504.0


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_f16(x):
    """IEEE fp32 -> fp16, round to nearest even (overflow -> inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def f32_to_f16_sat(x):
    """fp32 -> fp16 RNE, then clamp infinities to +-65504 (NaN is kept)."""
    h = f32_to_f16(x)
    h = np.where(np.isposinf(h), np.float16(F16_MAX), h)
    h = np.where(np.isneginf(h), np.float16(-F16_MAX), h)
    return h.astype(np.float16)


def f16_next_up(h):
    """Next fp16 value above positive finite h (by bit pattern)."""
    b = np.asarray(h, dtype=np.float16).view(np.uint16)
    return (b + np.uint16(1)).astype(np.uint16).view(np.float16)


def f16_next_down(h):
    b = np.asarray(h, dtype=np.float16).view(np.uint16)
    return (b - np.uint16(1)).astype(np.uint16).view(np.float16)


def f16_rne_sqrt_exact(ms):
    """fp16 RNE of sqrt(ms), exact, for non-negative fp64 ``ms``.

    The fp16 value h is the correctly rounded square root when the midpoints
    m- < h < m+ that bound its rounding interval satisfy m-^2 <= ms <= m+^2,
    with ties (ms equal to a squared midpoint) going to the even significand.
    A midpoint has at most 12 significant bits, so its square is exact in fp64
    and every comparison is exact.  Results at or above the fp16 overflow
    threshold (65520) saturate to 65504.
    """
    ms = np.asarray(ms, dtype=np.float64)
    if np.any(np.isnan(ms)) or np.any(ms < 0):
        raise ValueError("mean square must be a non-negative number")
    with np.errstate(over="ignore"):
        h = np.sqrt(ms).astype(np.float16)          # candidate (fp64 -> fp16)
    h = np.where(np.isinf(h), np.float16(F16_MAX), h).astype(np.float16)
    for _ in range(3):                               # exact correction
        hv = h.astype(np.float64)
        with np.errstate(over="ignore", invalid="ignore"):
            up = f16_next_up(h).astype(np.float64)   # inf above 65504
            mid_up = (hv + up) / 2.0
            dn = np.where(hv > 0, f16_next_down(np.where(hv > 0, h, np.float16(1))).astype(np.float64), 0.0)
            mid_dn = np.where(hv > 0, (dn + hv) / 2.0, -np.inf)
            odd = (h.view(np.uint16) & 1) == 1
            go_up = (ms > mid_up * mid_up) | ((ms == mid_up * mid_up) & odd)
            go_dn = (hv > 0) & ((ms < mid_dn * mid_dn) | ((ms == mid_dn * mid_dn) & odd))
        if not (go_up.any() or go_dn.any()):
            break
        h = np.where(go_up, f16_next_up(h), np.where(go_dn, f16_next_down(np.where(hv > 0, h, np.float16(1))), h))
        h = h.astype(np.float16)
    return h


# ---------------------------------------------------------------------------
# OCP FP8 e4m3fn
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Decode e4m3fn bytes to fp64: s eeee mmm, bias 7; e=0 is subnormal
    (m * 2^-9); 0x7F / 0xFF are NaN; there are no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def e4m3_encode(x):
    """fp32 -> e4m3fn, round to nearest even, saturating to +-448.

    The magnitude is rounded on the grid of its binade (spacing 2^(e-3) for
    e >= -6, 2^-9 below), which is an exact division by a power of two
    followed by round-half-even.  NaN -> 0x7F.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)
    q = np.rint(a / step) * step               # RNE on the binade grid
    q = np.minimum(q, E4M3_MAX)                # saturate to finite
    code = np.zeros(x.shape, dtype=np.int64)
    sub = q < 2.0 ** -6
    code = np.where(sub, np.rint(q / 2.0 ** -9).astype(np.int64), code)
    with np.errstate(divide="ignore"):
        qe = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    mant = np.rint((q / np.exp2(qe) - 1.0) * 8.0).astype(np.int64)
    norm_code = ((qe.astype(np.int64) + 7) << 3) | mant
    code = np.where(sub, code, norm_code)
    code = np.where(sign, code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# OCP FP4 e2m1 and the UE8M0 shared exponent
# ---------------------------------------------------------------------------

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """4-bit e2m1 code (sign bit 3) -> fp64 value."""
    c = np.asarray(codes).astype(np.int64)
    v = E2M1_VALUES[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode(x):
    """Real value (already divided by its block scale; fp32 or fp64) -> e2m1 code.

    Nearest grid value, ties to the even code (the code's low bit is the
    mantissa bit), magnitudes above 6 saturate to 6.  The sign bit is the
    input's sign bit, so small negative inputs give -0 (code 8).
    """
    x = np.asarray(x).astype(np.float64)
    a = np.abs(x)
    d = np.abs(a[..., None] - E2M1_VALUES)          # distance to all 8 values
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # ties: prefer the even code (mantissa bit 0)
    even = (np.arange(8) % 2) == 0
    pick = np.where((cand & even).any(axis=-1), np.argmax(cand & even, axis=-1), np.argmax(cand, axis=-1))
    pick = np.where(a >= 6.0, 7, pick)
    code = pick.astype(np.int64) | np.where(np.signbit(x), 8, 0)
    return code.astype(np.uint8)


def ue8m0_exponent(amax):
    """Shared exponent X of a 32-element block: floor(log2(amax)) - 2, the
    largest e2m1 exponent being 2, clamped to [-127, 127]; amax == 0 -> -127.

    ``amax`` is an fp32 magnitude, so floor(log2) is read exactly from its
    exponent field (math.frexp), subnormals included.
    """
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    out = np.empty(a.shape, dtype=np.int64)
    fa = a.reshape(-1)
    fo = out.reshape(-1)
    for i, v in enumerate(fa):
        if v == 0.0:
            fo[i] = -127
        else:
            m, e = math.frexp(v)            # v = m * 2^e, m in [0.5, 1)
            fo[i] = max(-127, min(127, (e - 1) - 2))
    return out
