"""GPU parity of the calibrated key-table fit against the CPU oracle, through
the C ABI: fitted fp16 tables bit for bit, fp64 levels and the per-layer MSEs
to 1e-10 relative (the sums run in another order), Lloyd update counts and the
choice of layers exactly; a fitted table then drives the TQ4/4 path."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import Case, check_case, say, to_dev_bf16
from oracle import calibrate, lloyd_max

pytestmark = pytest.mark.gpu

REL = 1e-10


def _gpu_fit(kbits, init=None, max_iters=100):
    from bit_quantized_kv_amd import calibrate_key_tables
    k = to_dev_bf16(kbits)
    tables, levels, mse, updates = calibrate_key_tables(k, init, max_iters)
    torch.cuda.synchronize()
    return (tables.cpu().numpy().view(np.uint16), levels.cpu().numpy(), mse.cpu().numpy(),
            updates.cpu().numpy())


def _oracle_fit(kbits, init_f16, max_iters=100):
    k = workloads.bf16_bits_to_f32(kbits)
    tabs, levs, mses, ups = [], [], [], []
    for layer in range(k.shape[0]):
        t, lv, n = calibrate.fit_table(k[layer], init_f16, max_iters)
        tabs.append(t.view(np.uint16))
        levs.append(lv)
        mses.append([calibrate.key_mse(k[layer], init_f16), calibrate.key_mse(k[layer], t)])
        ups.append(n)
    return np.array(tabs), np.array(levs), np.array(mses), np.array(ups)


def _compare(kbits, init=None, max_iters=100):
    init_f16 = (lloyd_max.default_key_table_f16() if init is None
                else np.asarray(init, np.float32).astype(np.float16))
    g = _gpu_fit(kbits, init, max_iters)
    o = _oracle_fit(kbits, init_f16, max_iters)
    assert np.array_equal(g[3], o[3]), f"updates {g[3]} vs {o[3]}"
    assert np.array_equal(g[0], o[0]), "fitted fp16 tables differ"
    np.testing.assert_allclose(g[1], o[1], rtol=REL, atol=1e-300)
    np.testing.assert_allclose(g[2], o[2], rtol=REL, atol=1e-300)
    return g, o


def test_full_stack_of_32_layers():
    kbits = workloads.calibration_keys()
    say(f"case: calibration 32 layers x {kbits.shape[1]} rows x D {kbits.shape[2]}, 100 iterations")
    g, o = _compare(kbits)
    from bit_quantized_kv_amd import tq_select_layers
    chosen = tq_select_layers(g[2][:, 0].tolist())
    assert chosen == calibrate.select_layers(o[2][:, 0]).tolist()
    assert sum(chosen) == 4
    say(f"  mse ratio fitted/initial {np.round(g[2][:, 1] / g[2][:, 0], 3).tolist()}")


def test_d64_ragged_rows_with_zero_and_tiny_rows():
    kbits = workloads.calibration_keys(layers=3, tokens=7, num_kv_heads=3, head_dim=64, seed=77)
    kbits[1, 4] = 0                                              # all-zero row
    kbits[2, 9] = workloads.f32_to_bf16_bits(np.full(64, 1e-9, np.float32))  # scale rounds to 0
    say("case: calibration D 64, 21 rows, a zero row and a row whose scale rounds to 0")
    _compare(kbits, max_iters=300)


def test_edge_cases():
    kb = workloads.calibration_keys(layers=2, tokens=3, num_kv_heads=1, head_dim=128, seed=78)
    say("case: calibration max_iters 0, custom start, a single row, no rows")
    g, _ = _compare(kb, max_iters=0)
    assert np.array_equal(g[0], np.tile(lloyd_max.default_key_table_f16().view(np.uint16), (2, 1)))
    assert np.array_equal(g[2][:, 0], g[2][:, 1])
    _compare(kb, init=list(np.linspace(-2.5, 2.5, 16)), max_iters=50)
    _compare(kb[:, :1], max_iters=50)
    g = _gpu_fit(kb[:, :0], max_iters=50)
    assert np.array_equal(g[3], [0, 0]) and np.all(g[2] == 0.0)


def test_fitted_table_drives_the_cache():
    kbits = workloads.calibration_keys(layers=4, seed=79)
    g, _ = _compare(kbits)
    worst = int(np.argmax(g[2][:, 0]))
    table = g[0][worst].view(np.float16).astype(np.float32).tolist()
    cfg = workloads.small_config(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(40, 600),
                                 seed=114)
    say(f"case: TQ4/4 path with the table fitted on layer {worst}")
    check_case(Case(cfg, key_table=table))
