"""GPU: tq_decode_attention_noalloc (the fixed device scratch instead of a
caller workspace) gives the same output as tq_decode_attention, bit for bit,
and stays within the oracle tolerance; two calls in a row, the second on a
smaller input (the scratch still holds the first call's partials); sizes
beyond the scratch are refused on the host."""
import ctypes
import os

import numpy as np
import pytest
import torch

import workloads
from gpu_common import TOL, Case, row_rel_err, say, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu


def _both(case, split):
    from bit_quantized_kv_amd import binding as B
    c = case.cfg
    ranges = case.write_ranges()
    case.quantize(ranges)
    op = case.oracle_pool(ranges)
    ctx = case.w.context_lens_at(0)
    q = to_dev_bf16(case.w.query_bits(0))
    mx = int(max(1, ctx.max()))
    saved = os.environ.pop("TQ_SPLIT_BLOCKS", None)
    os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    try:
        ws_out = case.cache.decode(q, case.table_dev, to_dev_i32(ctx), mx, c.scale)
        na_out = torch.full_like(ws_out, float("nan"))
        B.tq_decode_attention_noalloc(case.cache.handle, q, na_out, case.table_dev, to_dev_i32(ctx), mx, c.scale)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("TQ_SPLIT_BLOCKS", None)
        if saved is not None:
            os.environ["TQ_SPLIT_BLOCKS"] = saved
    ws_out, na_out = ws_out.cpu().numpy(), na_out.cpu().numpy()
    assert np.array_equal(ws_out.view(np.uint32), na_out.view(np.uint32)), "outputs differ"
    rows = [(b, h) for b in range(c.batch) for h in range(c.num_q_heads)]
    ref = case.oracle_decode(op, rows)
    err = row_rel_err(np.array([na_out[b, h] for b, h in rows]), np.array([ref[b, h] for b, h in rows]))
    say(f"  no-alloc decode identical to the workspace call, max rel err {err:.2e}")
    assert err <= TOL


def test_noalloc_decode_two_calls_second_smaller():
    big = workloads.small_config(batch=5, num_q_heads=16, num_kv_heads=2, head_dim=128, ctx_range=(900, 3000),
                                 seed=501)
    say("case: no-alloc decode, 5 sequences up to 3000 tokens, 8-block splits")
    _both(Case(big), 8)
    small = workloads.small_config(batch=2, num_q_heads=8, num_kv_heads=1, head_dim=64, ctx_range=(40, 300),
                                   seed=502)
    say("case: no-alloc decode, 2 sequences up to 300 tokens, 4-block splits")
    _both(Case(small), 4)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    from bit_quantized_kv_amd import Cache, binding as B
    cache = Cache(0, 128, 8, 16)
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(t.data_ptr())
    # 256 sequences x 64 heads x 4 splits of 16384 tokens: 34 MB of partials
    st = B.LIB.tq_decode_attention_noalloc(cache.handle, p, p, 0, p, 1024, p, 256, 64, 16384,
                                           ctypes.c_float(0.088), ctypes.c_void_p(0))
    assert st == 4, B.LIB.tq_last_error().decode()
    assert b"fixed scratch" in B.LIB.tq_last_error()
    cache.close()
