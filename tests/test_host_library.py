"""CPU-only checks of the C-ABI library: it loads, exports every entry point
that include/tq.h declares, and its host logic (sizes, validation, the default
key table) behaves as documented.  No kernel is launched."""
import ctypes
import os
import re
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ensure_built():
    path = os.path.join(ROOT, "bit_quantized_kv_amd", "libtq.so")
    if not os.path.exists(path):
        sys.path.insert(0, ROOT)
        import __graft_entry__
        __graft_entry__._build_module().build()
    return path


def _declared():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    lib = ctypes.CDLL(_ensure_built())
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    from bit_quantized_kv_amd import binding
    assert sorted(binding.EXPORTS) == names


def test_record_and_pool_sizes():
    _ensure_built()
    import bit_quantized_kv_amd as T
    assert T.tq_record_bytes(T.TQ_FORMAT_TQ4, 128) == 2432
    assert T.tq_record_bytes(T.TQ_FORMAT_TQ4, 64) == 1184
    assert T.tq_record_bytes(T.TQ_FORMAT_TQ4V2, 128) == 1920
    assert T.tq_record_bytes(T.TQ_FORMAT_TQ4V2, 64) == 928
    assert T.tq_record_bytes(T.TQ_FORMAT_MXFP4, 128) == 2176
    assert T.tq_pool_bytes(T.TQ_FORMAT_TQ4, 128, 8, 2048) == 2432 * 8 * 2048


def test_default_key_table_matches_oracle():
    _ensure_built()
    import bit_quantized_kv_amd as T
    from oracle import lloyd_max
    ours = np.array(T.tq_default_key_table(), dtype=np.uint16)
    assert np.array_equal(ours, lloyd_max.default_key_table_f16().view(np.uint16))


@pytest.mark.parametrize("fmt,d,hkv,nblk,status", [
    (0, 96, 1, 1, 2),      # unsupported head_dim
    (1, 64, 1, 1, 2),      # MX-FP4 is head_dim 128 only
    (0, 128, 0, 1, 1),     # no kv heads
    (0, 128, 1, 0, 1),     # no blocks
    (7, 128, 1, 1, 1),     # unknown format
])
def test_descriptor_validation(fmt, d, hkv, nblk, status):
    _ensure_built()
    import bit_quantized_kv_amd as T
    with pytest.raises(T.TqError) as e:
        T.tq_pool_bytes(fmt, d, hkv, nblk)
    assert e.value.status == status


def test_key_table_validation_happens_before_any_device_call():
    _ensure_built()
    import bit_quantized_kv_amd as T
    bad = list(np.linspace(-2, 2, 16))
    bad[3], bad[4] = bad[4], bad[3]
    with pytest.raises(T.TqError) as e:
        T.tq_create_cache(T.TQ_FORMAT_TQ4, 128, 1, 4, key_table=bad)
    assert e.value.status == 1
    with pytest.raises(T.TqError) as e:
        T.tq_create_cache(T.TQ_FORMAT_TQ4, 128, 1, 4, key_table=[0.0] * 16)
    assert e.value.status == 1
    # strictly ascending but with two midpoints far closer than the bin grid allows
    tight = list(np.linspace(-3, 3, 16))
    tight[7], tight[8], tight[9] = 0.0, 5e-4, 1e-3     # midpoints 5e-4 apart
    with pytest.raises(T.TqError) as e:
        T.tq_create_cache(T.TQ_FORMAT_TQ4, 128, 1, 4, key_table=tight)
    assert e.value.status == 2
    with pytest.raises(T.TqError) as e:
        T.tq_create_cache(T.TQ_FORMAT_MXFP4, 128, 1, 4, key_table=list(range(16)))
    assert e.value.status == 1


def test_layer_choice_matches_oracle():
    _ensure_built()
    import bit_quantized_kv_amd as T
    from oracle import calibrate
    g = np.random.default_rng(3)
    for n in (0, 1, 7, 10, 30, 32, 64, 101):
        mse = g.random(n)
        if n > 4:
            mse[1] = mse[3]                      # a tie
        for pct in (0, 10, 25, 100):
            assert T.tq_select_layers(mse.tolist(), pct) == calibrate.select_layers(mse, pct).tolist()
    with pytest.raises(T.TqError):
        T.tq_select_layers([0.1, float("nan")])
    with pytest.raises(T.TqError):
        T.tq_select_layers([0.1], 101)


def test_calibration_sizes_and_validation():
    _ensure_built()
    import bit_quantized_kv_amd as T
    n = 32 * 160 * 128
    assert T.tq_calibrate_workspace_bytes(32, 160, 128) == n * 8 + n * 4 + 32 * 160 * 4
    assert T.tq_calibrate_workspace_bytes(0, 0, 64) == 0
    for args, status in (((1, 1, 96), 2), ((-1, 1, 128), 1), ((1, -1, 128), 1), ((1, 1 << 24, 128), 1)):
        with pytest.raises(T.TqError) as e:
            T.tq_calibrate_workspace_bytes(*args)
        assert e.value.status == status
