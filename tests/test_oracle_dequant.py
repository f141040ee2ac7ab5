"""Pins for oracle.paged.PagedPool.dequantize_blocks: hand-worked rows placed
at known (block, kv-head, token) positions come back at those positions with
the values worked out by hand (tests/golden/tq4_key_hand.json,
tq4_value_hand.json), and rows never written read as zero."""
import json
import os

import numpy as np

from oracle import lloyd_max, paged

HERE = os.path.dirname(__file__)
TABLE = lloyd_max.default_key_table_f16()


def _value_group(spec, pad):
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


def _codes(case):
    if isinstance(case["codes"], list):
        want = np.full(32, case.get("pad_code", 0))
        want[: len(case["codes"])] = case["codes"]
        return want
    if case["codes"].startswith("0 everywhere"):
        return np.zeros(32)
    return np.array([min(i, 15) for i in range(32)])


def test_tq4_rows_land_where_written_with_hand_values():
    vals = json.load(open(os.path.join(HERE, "golden", "tq4_value_hand.json")))["cases"]
    # D = 64, 2 kv-heads, 3 blocks; every hand value group goes into group 0 of
    # kv-head 1 at block 2, token row 4 + case index; group 1 is the constant
    # 3.25 (sc = 0, dequantizes to 3.25); keys are all ones (s = 1, codes 15
    # at channel 0 and 7 elsewhere: tq4_key_hand.json "all ones")
    pool = paged.PagedPool(paged.FORMAT_TQ4, 3, 2, 64)
    n = len(vals)
    k = np.ones((n, 2, 64), np.float32)
    v = np.zeros((n, 2, 64), np.float32)
    for i, case in enumerate(vals):
        v[i, 1, :32] = _value_group(case["v"], case.get("pad", 0.0))
        v[i, 1, 32:] = 3.25
    slots = 2 * 16 + 4 + np.arange(n)
    pool.append(k, v, slots)
    kh, vh = pool.dequantize_blocks([2, 0])
    assert kh.shape == (2, 2, 16, 64) and kh.dtype == np.float32
    assert np.all(kh[1] == 0) and np.all(vh[1] == 0)            # block 0 never written
    c15, c7 = float(TABLE[15]), float(TABLE[7])
    for i, case in enumerate(vals):
        t = 4 + i
        for h in (0, 1):
            assert kh[0, h, t, 0] == c15 and np.all(kh[0, h, t, 1:] == c7), case["name"]
        want = _codes(case) * case["sc"] + case["mn"]              # small exact hand values
        assert np.array_equal(vh[0, 1, t, :32], want.astype(np.float32)), case["name"]
        assert np.all(vh[0, 1, t, 32:] == 3.25), case["name"]
    untouched = [t for t in range(16) if not 4 <= t < 4 + n]
    assert np.all(kh[0][:, untouched] == 0) and np.all(vh[0][:, untouched] == 0)


def test_mxfp4_rows_land_where_written_with_hand_values():
    # values on the e2m1 grid with amax 6 (X = floor(log2 6) - 2 = 0) decode to
    # themselves; times 2^10 (X = 10) and 2^-30 (X = -30) exactly scaled
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, 6] * 2, np.float32)
    pool = paged.PagedPool(paged.FORMAT_MXFP4, 2, 1, 128)
    v = np.stack([np.concatenate([grid, grid * 2.0 ** 10, grid * 2.0 ** -30, -grid])])[:, None, :]
    k = np.zeros((1, 1, 128), np.float32)
    pool.append(k, v.astype(np.float32), np.array([16 + 9]))
    kh, vh = pool.dequantize_blocks([1])
    assert np.array_equal(vh[0, 0, 9], v[0, 0])
    assert np.all(kh[0, 0] == 0)
    assert np.all(vh[0, 0, :9] == 0) and np.all(vh[0, 0, 10:] == 0)
