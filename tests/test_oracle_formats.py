"""Pins for oracle.fpformats: torch's own conversions, exhaustive tables, ties."""
import numpy as np
import torch

from oracle import fpformats as fp
import workloads


def test_fp16_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 10.0 ** rng.integers(-8, 5, 200000),
                        np.array([65504.0, 65519.9, 65520.0, 1e-8, -6e-8, 0.0, -0.0], np.float32)]).astype(np.float32)
    ours = fp.f32_to_f16(x).view(np.uint16)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_fp16_saturating():
    h = fp.f32_to_f16_sat(np.array([1e6, -1e6, 70000.0, 65519.0], np.float32))
    assert list(h.astype(np.float64)) == [65504.0, -65504.0, 65504.0, 65504.0]


def test_bf16_generator_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(300000) * 10.0 ** rng.integers(-20, 20, 300000)).astype(np.float32)
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(fp.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_exact_sqrt_rounding_against_neighbours():
    rng = np.random.default_rng(3)
    allf = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    ms = np.concatenate([rng.random(50000) * 100.0, rng.random(5000) * 1e-9, allf ** 2, [0.0]])
    h = fp.f16_rne_sqrt_exact(ms).astype(np.float64)
    r = np.sqrt(ms)
    i = np.clip(np.searchsorted(allf, r), 1, len(allf) - 1)
    lo, hi = allf[i - 1], allf[i]
    best = np.where(np.abs(hi - r) < np.abs(lo - r), hi, lo)
    best = np.where(r >= allf[-1], allf[-1], best)
    assert np.array_equal(h, best)


def test_exact_sqrt_ties_and_saturation():
    # 1 + 2^-11 is the midpoint between 1 and 1 + 2^-10; its square as ms is a tie -> even (1.0)
    mid = 1.0 + 2.0 ** -11
    assert float(fp.f16_rne_sqrt_exact(np.array([mid * mid]))[0]) == 1.0
    # midpoint between 1 + 2^-10 (odd) and 1 + 2^-9 (even) -> 1 + 2^-9
    mid2 = 1.0 + 3 * 2.0 ** -11
    assert float(fp.f16_rne_sqrt_exact(np.array([mid2 * mid2]))[0]) == 1.0 + 2.0 ** -9
    # just above a tie rounds up
    assert float(fp.f16_rne_sqrt_exact(np.array([np.nextafter(mid * mid, 2.0)]))[0]) == 1.0 + 2.0 ** -10
    assert float(fp.f16_rne_sqrt_exact(np.array([1e12]))[0]) == 65504.0
    assert float(fp.f16_rne_sqrt_exact(np.array([0.0]))[0]) == 0.0


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == 448.0


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(400000) * 10.0 ** rng.uniform(-4, 2.6, 400000)).astype(np.float32)
    x = x[np.abs(x) < 464.0]
    # every midpoint between consecutive finite values is a tie case
    vals = np.unique(np.abs(fp.e4m3_decode(np.arange(0, 127, dtype=np.uint8))))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0])])
    ours = fp.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates():
    out = fp.e4m3_encode(np.float32([500.0, 1e30, -1e30, 448.0]))
    assert list(out) == [0x7E, 0x7E, 0xFE, 0x7E]


def test_e2m1_table_and_ties():
    assert list(fp.e2m1_decode(np.arange(8))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(fp.e2m1_decode(np.arange(8, 16))) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 5.01: 7, 6.0: 7, 7.9: 7, 100.0: 7,
             0.24: 0, 0.26: 1, -0.1: 8, -0.0: 8, -2.6: 13}
    for x, c in cases.items():
        assert int(fp.e2m1_encode(np.float64(x))) == c, x


def test_e2m1_nearest_bruteforce():
    x = np.linspace(-8, 8, 64001)
    codes = fp.e2m1_encode(x)
    vals = fp.e2m1_decode(codes)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    a = np.minimum(np.abs(x), 6.0)
    best = np.min(np.abs(a[:, None] - grid), axis=1)
    assert np.allclose(np.abs(np.minimum(np.abs(vals), 6) - a), best)
    assert np.all(np.signbit(vals) == np.signbit(x))


def test_ue8m0_exponent():
    for e in range(-126, 127):
        a = np.float32(2.0 ** e)
        assert int(fp.ue8m0_exponent(a)) == max(-127, min(127, e - 2))
        b = np.float32(2.0 ** e * 1.999)
        assert int(fp.ue8m0_exponent(b)) == max(-127, min(127, e - 2))
    assert int(fp.ue8m0_exponent(np.float32(0.0))) == -127
    assert int(fp.ue8m0_exponent(np.float32(2.0 ** -140))) == -127   # subnormal, clamped
