"""Pins for oracle.tq4: centroid round trip, exact-rule agreement, hand cases."""
import json
import os

import numpy as np
import pytest

from oracle import lloyd_max, tq4, wht
import workloads

HERE = os.path.dirname(__file__)
TABLE = lloyd_max.default_key_table_f16()


def _expand_codes(spec, d):
    out = np.full(d, spec.get("rest", -1))
    if "even" in spec:
        out[0::2] = spec["even"]
    if "odd" in spec:
        out[1::2] = spec["odd"]
    for k, v in spec.items():
        if k.isdigit():
            out[int(k)] = v
    return out


def test_hand_keys():
    g = json.load(open(os.path.join(HERE, "golden", "tq4_key_hand.json")))
    for case in g["cases"]:
        k = np.zeros(64, np.float32)
        if "all" in case["k"]:
            k[:] = case["k"]["all"]
        for idx, val in case["k"].items():
            if idx.isdigit():
                k[int(idx)] = val
        s = tq4.key_scale(k[None])[0]
        assert float(s) == case["s"], case["name"]
        codes = tq4.key_codes(k[None], np.array([s]), TABLE)[0]
        assert np.array_equal(codes, _expand_codes(case["codes"], 64)), case["name"]
        ex, _ = tq4.key_codes_exact(k[None], np.array([s]), TABLE)
        assert np.array_equal(ex[0], codes), case["name"]


def test_centroid_round_trip():
    """u = c_j * s * fp32(1/s) must code back to j, for every entry and many scales."""
    rng = np.random.default_rng(9)
    s = np.unique(rng.uniform(1e-3, 300.0, 2000).astype(np.float16))
    s = s[s > 0].astype(np.float32)
    c = TABLE.astype(np.float32)
    y = (c[None, :] * s[:, None]).astype(np.float32)                 # exact
    inv = (np.float32(1.0) / s).astype(np.float32)
    u = (y * inv[:, None]).astype(np.float32)
    codes = tq4.key_codes_from_units(u, TABLE)
    assert np.array_equal(codes, np.broadcast_to(np.arange(16), codes.shape))


def test_dequant_then_nearest_is_fixed_point():
    rng = np.random.default_rng(10)
    codes = rng.integers(0, 16, size=(100, 128)).astype(np.uint8)
    s = rng.uniform(0.1, 10, 100).astype(np.float16)
    kh = tq4.key_dequant_rot(codes, s, TABLE)
    u = kh / s.astype(np.float32)[:, None]
    assert np.array_equal(tq4.key_codes_from_units(u, TABLE), codes)


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_rule_matches_exact_rule_away_from_near_ties(d):
    cfg = workloads.small_config(head_dim=d, batch=2, ctx_range=(600, 600), num_kv_heads=4, seed=11)
    w = workloads.make(cfg)
    k = workloads.bf16_bits_to_f32(w.sequence_kv(0)[0]).reshape(-1, d)
    s = tq4.key_scale(k)
    fast = tq4.key_codes(k, s, TABLE)
    exact, near = tq4.key_codes_exact(k, s, TABLE)
    mism = fast != exact
    assert not np.any(mism & ~near)
    assert near.mean() < 1e-3


def test_scale_is_exact_rms_and_rotation_invariant():
    rng = np.random.default_rng(12)
    k = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal((500, 128)).astype(np.float32) * 3))
    s = tq4.key_scale(k).astype(np.float64)
    rms = np.sqrt(np.mean(k.astype(np.float64) ** 2, axis=1))
    # s is the fp16 value nearest to the RMS
    assert np.all(np.abs(s - rms) <= np.abs(np.float16(rms).astype(np.float64) - rms) + 1e-12)
    rms_rot = np.sqrt(np.mean(wht.wht_f64(k) ** 2, axis=1))
    assert np.allclose(rms, rms_rot, rtol=1e-13)


def test_power_of_two_scale_invariance():
    rng = np.random.default_rng(13)
    k = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal((300, 64)).astype(np.float32)))
    s = tq4.key_scale(k)
    c1 = tq4.key_codes(k, s, TABLE)
    for e in (-3, 4):
        k2 = (k * np.float32(2.0 ** e)).astype(np.float32)
        s2 = tq4.key_scale(k2)
        assert np.array_equal(s2.astype(np.float64), s.astype(np.float64) * 2.0 ** e)
        assert np.array_equal(tq4.key_codes(k2, s2, TABLE), c1)


def test_zero_and_saturated_keys():
    k = np.zeros((1, 128), np.float32)
    s = tq4.key_scale(k)
    assert float(s[0]) == 0.0
    assert np.all(tq4.key_codes(k, s, TABLE) == 7)
    assert np.all(tq4.key_dequant_rot(tq4.key_codes(k, s, TABLE), s, TABLE) == 0)
    big = np.full((1, 128), 1e6, np.float32)
    assert float(tq4.key_scale(big)[0]) == 65504.0


def test_key_quantization_mse_on_gaussian_rows():
    """Rotated N(0,1) keys: normalized per-element error close to the
    Lloyd-Max value 0.0095 (a quality report, not parity)."""
    rng = np.random.default_rng(14)
    k = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal((4000, 128)).astype(np.float32)))
    s = tq4.key_scale(k)
    codes = tq4.key_codes(k, s, TABLE)
    y = wht.wht_f64(k)
    err = y - tq4.key_dequant_rot(codes, s, TABLE)
    nmse = np.mean(err ** 2) / np.mean(y ** 2)
    assert 0.0085 < nmse < 0.0105


def _group_from_spec(spec, pad):
    if isinstance(spec, list):
        v = np.full(32, pad, np.float32)
        v[: len(spec)] = spec
        return v
    if spec.startswith("i for i < 16, then 15"):
        return np.array([min(i, 15) for i in range(32)], np.float32)
    if spec.startswith("-1 + 0.5 i"):
        return np.array([-1 + 0.5 * min(i, 15) for i in range(32)], np.float32)
    if spec.startswith("3.25"):
        return np.full(32, 3.25, np.float32)
    raise ValueError(spec)


def test_hand_value_groups():
    g = json.load(open(os.path.join(HERE, "golden", "tq4_value_hand.json")))
    for case in g["cases"]:
        v = _group_from_spec(case["v"], case.get("pad", 0.0))
        codes, sc, mn = tq4.value_encode(v[None])
        assert float(sc[0, 0]) == case["sc"], case["name"]
        assert float(mn[0, 0]) == case["mn"], case["name"]
        if isinstance(case["codes"], list):
            want = np.full(32, case.get("pad_code", 0))
            want[: len(case["codes"])] = case["codes"]
        elif case["codes"].startswith("0 everywhere"):
            want = np.zeros(32)
        else:
            want = np.array([min(i, 15) for i in range(32)])
        assert np.array_equal(codes[0], want), case["name"]
        ex, _ = tq4.value_codes_exact(v[None], sc, mn)
        assert np.array_equal(ex[0], codes[0]), case["name"]
    # constant group dequantizes to its minimum
    c, sc, mn = tq4.value_encode(np.full((1, 32), 3.25, np.float32))
    assert np.all(tq4.value_dequant(c, sc, mn) == np.float32(3.25))


def test_value_rule_bounds_idempotence_and_exactness():
    cfg = workloads.small_config(batch=1, ctx_range=(2000, 2000), num_kv_heads=2, seed=15)
    w = workloads.make(cfg)
    v = workloads.bf16_bits_to_f32(w.sequence_kv(0)[1]).reshape(-1, 128)
    codes, sc, mn = tq4.value_encode(v)
    vh = tq4.value_dequant(codes, sc, mn).astype(np.float64)
    g = lambda a: a.reshape(a.shape[0], 4, 32)
    sc64 = sc.astype(np.float64)[..., None]
    bound = sc64 / 2 + np.abs(v.reshape(-1, 4, 32).min(-1, keepdims=True) - mn.astype(np.float64)[..., None]) + 1e-6
    assert np.all(np.abs(g(v.astype(np.float64)) - g(vh)) <= bound + sc64 * 1e-3)
    assert np.array_equal(tq4.value_codes(vh.astype(np.float32), sc, mn), codes)
    ex, near = tq4.value_codes_exact(v, sc, mn)
    assert not np.any((ex != codes) & ~near)


def test_hand_value_groups_2bit():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tq4_value2_hand.json")))
    for case in g["cases"]:
        v = np.full(32, case["pad"], dtype=np.float32)
        v[:len(case["v"])] = case["v"]
        codes, sc, mn = tq4.value_encode(v[None], levels=3)
        assert float(sc[0, 0]) == case["sc"], case["name"]
        assert float(mn[0, 0]) == case["mn"], case["name"]
        want = np.full(32, case["pad_code"], dtype=np.uint8)
        want[:len(case["codes"])] = case["codes"]
        assert np.array_equal(codes[0], want), case["name"]


def test_2bit_value_rule_bounds_and_exactness():
    rng = np.random.default_rng(40)
    v = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal((500, 128)).astype(np.float32)))
    codes, sc, mn = tq4.value_encode(v, levels=3)
    assert codes.max() <= 3
    ex, near = tq4.value_codes_exact(v, sc, mn, levels=3)
    assert np.array_equal(codes[~near], ex[~near])
    vh = tq4.value_dequant(codes, sc, mn)
    g = lambda a: a.reshape(500, 4, 32)
    # inside the group's range the error is at most half a step (plus fp16 rounding of sc, mn)
    err = np.abs(g(vh) - g(v)).max(-1)
    assert np.all(err <= sc.astype(np.float64) * 0.5 * (1 + 1e-2) + np.abs(mn.astype(np.float64)) * 2 ** -10 + 1e-6)
    # the group's extremes are reproduced up to the fp16 roundings
    assert np.all(np.abs(g(vh).min(-1) - mn.astype(np.float64)) <= 1e-6)
