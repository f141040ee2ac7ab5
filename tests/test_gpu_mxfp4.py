"""GPU parity of the MX-FP4 path (FP4 e2m1 K/V with UE8M0 group exponents,
FP8 e4m3 queries, scaled MFMA) against the CPU oracle, through the C ABI.

Packed bytes must be identical; decode attention must be within 2e-3 (max over
rows of ||o - o_ref||_inf / ||o_ref||_inf) of the oracle's fp64 attention over
the same dequantized cache with the same e4m3 query."""
import os

import numpy as np
import pytest
import torch

import workloads
from gpu_common import TOL, Case, describe_record_diff, row_rel_err, say, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _split_env():
    old = os.environ.pop("TQ_SPLIT_BLOCKS", None)
    yield
    os.environ.pop("TQ_SPLIT_BLOCKS", None)
    if old is not None:
        os.environ["TQ_SPLIT_BLOCKS"] = old


def _check(case, seqs=None, rows=None):
    c = case.cfg
    seqs = list(range(c.batch)) if seqs is None else seqs
    ranges = case.write_ranges()
    case.quantize(ranges)
    gpu = case.pool_np()
    op = case.oracle_pool([r for r in ranges if r[0] in seqs])
    blocks = case.blocks_of(seqs)
    mism = np.nonzero(np.any(gpu[blocks] != op.pool[blocks], axis=-1))
    if mism[0].size:
        bi, hi = blocks[mism[0][0]], mism[1][0]
        raise AssertionError(f"{mism[0].size} records differ; block {bi} head {hi}: "
                             + describe_record_diff(gpu[bi, hi], op.pool[bi, hi], 128, 1))
    out = case.decode()
    rows = rows if rows is not None else [(b, h) for b in seqs for h in range(c.num_q_heads)]
    ref = case.oracle_decode(op, rows)
    err = row_rel_err(np.array([out[b, h] for b, h in rows]), np.array([ref[b, h] for b, h in rows]))
    say(f"  {c.name}: {len(blocks)} blocks byte-identical, {len(rows)} rows, max rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("g,hkv,seed,split", [(8, 1, 201, None), (4, 2, 202, 4), (1, 2, 203, None), (2, 3, 204, 12)])
def test_small_ragged_fp4(g, hkv, seed, split):
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=5, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=128, ctx_range=(1, 700),
                                 seed=seed, fmt=1)
    say(f"case: fp4 small ragged g={g} hkv={hkv} seed={seed} split={split}")
    _check(Case(cfg))


@pytest.mark.parametrize("loop", ["static", "balanced", "balanced-pairs"])
def test_fp4_both_quantize_loops(loop):
    """Every work distribution of the quantize kernel writes the oracle's bytes."""
    saved = os.environ.get("TQ_QUANT_LOOP")
    os.environ["TQ_QUANT_LOOP"] = loop
    try:
        cfg = workloads.small_config(batch=6, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(1500, 3000),
                                     seed=231, fmt=1)
        say(f"case: fp4 quantize loop {loop}")
        _check(Case(cfg))
    finally:
        os.environ.pop("TQ_QUANT_LOOP", None)
        if saved is not None:
            os.environ["TQ_QUANT_LOOP"] = saved


def test_fp4_unaligned_skipped_single_token_slots():
    cfg = workloads.small_config(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=128, ctx_range=(160, 160),
                                 seed=205, fmt=1)
    w = workloads.make(cfg)
    from bit_quantized_kv_amd import Cache
    from oracle import paged
    k, v = w.sequence_kv(0)
    rng = np.random.default_rng(6)
    slots = rng.permutation(w.num_blocks * 16)[:160].astype(np.int32)
    slots[rng.choice(160, 20, replace=False)] = -1
    cache = Cache(1, 128, 2, w.num_blocks)
    say("case: fp4 permuted slots with skips, then one-token appends")
    cache.quantize_append(to_dev_bf16(k[:100]), to_dev_bf16(v[:100]), to_dev_i32(slots[:100]))
    for i in range(100, 160):
        cache.quantize_append(to_dev_bf16(k[i:i + 1]), to_dev_bf16(v[i:i + 1]), to_dev_i32(slots[i:i + 1]))
    torch.cuda.synchronize()
    gpu = cache.pool.cpu().numpy().reshape(w.num_blocks, 2, -1)
    op = paged.PagedPool(1, w.num_blocks, 2, 128)
    op.append(workloads.bf16_bits_to_f32(k), workloads.bf16_bits_to_f32(v), slots)
    assert np.array_equal(gpu, op.pool)


def test_fp4_edge_lengths():
    cfg = workloads.small_config(batch=6, num_q_heads=8, num_kv_heads=1, head_dim=128, ctx_range=(40, 60), seed=206,
                                 fmt=1)
    case = Case(cfg)
    ranges = case.write_ranges()
    case.quantize(ranges)
    op = case.oracle_pool(ranges)
    ctx = np.array([0, 1, 15, 16, 17, 33], np.int32)
    say(f"case: fp4 edge lengths {ctx.tolist()}")
    out = case.decode(ctx=ctx)
    rows = [(b, h) for b in range(6) for h in range(8)]
    ref = case.oracle_decode(op, rows, ctx=ctx)
    assert np.all(out[0] == 0)
    assert row_rel_err(out, ref) <= TOL


def test_full_fp4_sampled():
    say("case: fp4 (B=128, 64/8, D=128, T=16384), sampled sequences")
    _check(Case(workloads.CONFIGS["fp4"]), seqs=[0, 77, 127], rows=[(b, h) for b in (0, 77, 127) for h in range(64)])


def test_one_query_token_multi_token_matches_decode():
    """One query token per sequence through the MX-FP4 multi-token kernel
    equals the MX-FP4 decode kernel up to summation order: both take the
    logits from the same scaled MFMA and P as bf16 high + low parts."""
    cfg = workloads.small_config(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(50, 900),
                                 fmt=1, seed=141)
    case = Case(cfg)
    case.quantize(case.write_ranges())
    w = case.w
    qbits, q_start = w.multi_queries(1)
    ctx = w.total_lens.astype(np.int32)
    say("case: MX-FP4 multi-token with one query token per sequence against decode")
    mt = case.cache.multitoken(to_dev_bf16(qbits), to_dev_i32(q_start), 1, case.table_dev, to_dev_i32(ctx),
                               int(ctx.max()), cfg.scale)
    dec = case.cache.decode(to_dev_bf16(qbits), case.table_dev, to_dev_i32(ctx), int(ctx.max()), cfg.scale)
    torch.cuda.synchronize()
    assert row_rel_err(mt.cpu().numpy(), dec.cpu().numpy()) <= 1e-4
