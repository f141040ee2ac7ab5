"""GPU: the dequantized cache that the attention kernels consume is bit-exact.

tq_debug_dequantize writes, through the decode kernels' own record reader and
dequantization routines, the fp32 k_hat (rotated domain) and v_hat of whole
records; they must equal the oracle's definitions bit for bit
(oracle.paged.PagedPool.dequantize_blocks: k_hat = c[code] * s, v_hat =
fp32(code * sc + mn), MX-FP4 e2m1 * 2^X), for every row of every record,
including the unwritten rows of partial last blocks.  The range edges (value
groups beyond the fp16 range, tiny values, big queries, tiny keys) are checked
the same way and through decode attention against the oracle at 2e-3."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import TOL, Case, row_rel_err, say, to_dev_i32

pytestmark = pytest.mark.gpu


def _all_block_ids(case):
    return np.arange(case.w.num_blocks, dtype=np.int32)


def _check_bits(case, op, ids, label):
    kg, vg = case.cache.dequantize(to_dev_i32(ids))
    torch.cuda.synchronize()
    kg, vg = kg.cpu().numpy(), vg.cpu().numpy()
    ko, vo = op.dequantize_blocks(ids)
    for name, g, o in (("k", kg, ko), ("v", vg, vo)):
        gb, ob = g.view(np.uint32), o.view(np.uint32)
        bad = np.argwhere(gb != ob)
        if bad.size:
            i = tuple(bad[0])
            raise AssertionError(f"{label}: {len(bad)} {name} elements differ; first at (block {ids[i[0]]}, "
                                 f"head {i[1]}, row {i[2]}, channel {i[3]}): gpu {g[i]!r} oracle {o[i]!r}")
    say(f"  {label}: {kg.size} key and {vg.size} value elements bit-identical")


def _quantize_both(cfg):
    case = Case(cfg)
    ranges = case.write_ranges()
    case.quantize(ranges)
    op = case.oracle_pool(ranges)
    gpu = case.pool_np()
    assert np.array_equal(gpu, op.pool), "packed records differ from the oracle's"
    return case, op


@pytest.mark.parametrize("fmt,d,hkv,g,seed", [
    (0, 128, 2, 4, 301), (0, 64, 3, 2, 302), (2, 128, 2, 8, 303), (2, 64, 1, 4, 304), (1, 128, 2, 8, 305),
])
def test_dequantize_bit_exact(fmt, d, hkv, g, seed):
    cfg = workloads.small_config(batch=4, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                                 ctx_range=(1, 300), fmt=fmt, seed=seed)
    say(f"case: dequantize fmt={fmt} d={d} hkv={hkv} seed={seed}")
    case, op = _quantize_both(cfg)
    ids = _all_block_ids(case)
    # every record, the partly written last blocks' empty rows included, and
    # the same ids again in another order
    _check_bits(case, op, ids, "all records")
    _check_bits(case, op, ids[::-1].copy(), "reversed ids")


def _decode_parity(case, op, label):
    c = case.cfg
    out = case.decode()
    rows = [(b, h) for b in range(c.batch) for h in range(c.num_q_heads)]
    ref = case.oracle_decode(op, rows)
    err = row_rel_err(np.array([out[b, h] for b, h in rows]), np.array([ref[b, h] for b, h in rows]))
    say(f"  {label}: decode max rel err {err:.2e}")
    assert np.all(np.isfinite(out))
    assert err <= TOL


@pytest.mark.parametrize("fmt,v_scale,seed", [
    (0, 3.0e4, 311),      # groups spanning > 65520: scales >= 4096, saturated minima
    (0, 1.0e5, 312),
    (2, 3.0e4, 313),      # 2-bit values: scales up to ~(2 * 65504) / 3
    (0, 1.0e-6, 314),     # tiny values: fp16-subnormal scales and minima
    (2, 1.0e-6, 315),
    (1, 2.0 ** 18, 316),  # MX-FP4 groups with amax >= 2^16 (X >= 14)
    (1, 2.0 ** -30, 317), # and amax <= 2^-24
])
def test_value_range_edges(fmt, v_scale, seed):
    cfg = workloads.small_config(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(20, 400),
                                 fmt=fmt, seed=seed, v_scale=v_scale)
    say(f"case: value range fmt={fmt} v_scale={v_scale:g} seed={seed}")
    case, op = _quantize_both(cfg)
    _check_bits(case, op, _all_block_ids(case), f"v x {v_scale:g}")
    _decode_parity(case, op, f"v x {v_scale:g}")


@pytest.mark.parametrize("fmt,k_scale,q_scale,seed", [
    (0, 1.0, 1.0e4, 321),    # large queries: rotated query near the fp16 range
    (0, 1.0e-6, 1.0, 322),   # all-tiny keys: fp16-subnormal key scales
    (2, 1.0e-6, 1.0, 323),
])
def test_key_and_query_range_edges(fmt, k_scale, q_scale, seed):
    cfg = workloads.small_config(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(20, 400),
                                 fmt=fmt, seed=seed, k_scale=k_scale, q_scale=q_scale)
    say(f"case: key/query range fmt={fmt} k_scale={k_scale:g} q_scale={q_scale:g} seed={seed}")
    case, op = _quantize_both(cfg)
    _check_bits(case, op, _all_block_ids(case), f"k x {k_scale:g}")
    _decode_parity(case, op, f"k x {k_scale:g}, q x {q_scale:g}")
