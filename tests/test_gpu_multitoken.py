"""GPU parity of multi-token attention over the TQ4/4, TQ4/2 and MX-FP4 caches
(chunked prefill, verification) against the CPU oracle, through the C ABI: max over rows of
||o - o_ref||_inf / ||o_ref||_inf within 2e-3, rows computed by the oracle's
exact fp64 causal attention over the same (byte-identical) cache."""
import os

import numpy as np
import pytest
import torch

import workloads
from gpu_common import TOL, Case, row_rel_err, say, to_dev_bf16, to_dev_i32
from oracle import attention

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _split_env():
    saved = os.environ.pop("TQ_SPLIT_BLOCKS", None)
    yield
    os.environ.pop("TQ_SPLIT_BLOCKS", None)
    if saved is not None:
        os.environ["TQ_SPLIT_BLOCKS"] = saved


def _run(case, m, rows=None, seqs=None):
    """Quantize the workload, run multi-token attention for ``m`` query tokens
    per sequence, compare ``rows`` (or all) with the oracle."""
    c = case.cfg
    w = case.w
    ranges = case.write_ranges(w.total_lens)
    case.quantize(ranges)
    gpu_pool = case.pool_np()
    seqs = list(range(c.batch)) if seqs is None else seqs
    writer = w.prefix_writer()
    op = case.oracle_pool([r for r in ranges if r[0] in seqs or r[0] == writer])
    blocks = case.blocks_of(seqs)
    assert np.array_equal(gpu_pool[blocks], op.pool[blocks]), "cache records differ from the oracle's"
    qbits, q_start = w.multi_queries(m)
    mq = int(np.max(np.diff(q_start))) if c.batch else 0
    ctx = w.total_lens.astype(np.int32)
    out = case.cache.multitoken(to_dev_bf16(qbits), to_dev_i32(q_start), max(mq, 1), case.table_dev,
                                to_dev_i32(ctx), int(ctx.max()), c.scale)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    if rows is None:
        rows = [(i, h) for b in seqs for i in range(int(q_start[b]), int(q_start[b + 1]))
                for h in range(c.num_q_heads)]
    q = workloads.bf16_bits_to_f32(qbits)
    ref = attention.multi_token(op, q, q_start, w.block_table, ctx, c.scale, rows=rows)
    o = np.array([out[i, h] for i, h in rows])
    r = np.array([ref[i, h] for i, h in rows])
    err = row_rel_err(o, r)
    say(f"  {c.name}: {len(rows)} rows, max rel err {err:.2e}")
    assert err <= TOL
    return out, q_start


@pytest.mark.parametrize("d,g,hkv,seed,mmax,split", [
    (128, 4, 2, 201, 40, None), (128, 8, 1, 202, 20, 8), (128, 1, 2, 203, 150, None), (128, 2, 3, 204, 70, 12),
    (64, 4, 2, 205, 40, None), (64, 8, 1, 206, 33, 4), (64, 1, 1, 207, 130, 16),
])
def test_small_ragged(d, g, hkv, seed, mmax, split):
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=5, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                                 ctx_range=(1, 700), seed=seed)
    rng = np.random.default_rng(seed)
    m = rng.integers(1, mmax + 1, size=5)
    say(f"case: multi-token small ragged d={d} g={g} hkv={hkv} seed={seed} m={m.tolist()} split={split}")
    _run(Case(cfg), m)


@pytest.mark.parametrize("d,g,hkv,seed,m,split", [
    (128, 4, 2, 221, [3, 8, 1, 5, 8], None),       # at most 32 rows: the direct kernel, two row tiles
    (128, 8, 1, 222, [2, 1, 2, 0, 2], None),       # at most 16 rows: the direct kernel, one row tile
    (128, 8, 1, 223, [8, 3, 5, 7, 1], 8),          # 64 rows: the staged kernel, 8-block splits
    (128, 4, 2, 224, [30, 12, 1, 25, 9], None),    # 120 rows: the staged kernel, 128-row tiles
    (64, 8, 1, 225, [32, 5, 17, 1, 26], 16),       # 256 rows at D = 64
    (64, 2, 2, 226, [16, 4, 9, 1, 12], None),      # 32 rows at D = 64: the direct kernel
])
def test_two_bit_values(d, g, hkv, seed, m, split):
    """TQ4/2 caches (2-bit values) through both kernels and every row tiling."""
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=5, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                                 ctx_range=(60, 700), seed=seed, fmt=2)
    say(f"case: multi-token TQ4/2 d={d} g={g} hkv={hkv} seed={seed} m={m} split={split}")
    _run(Case(cfg), np.array(m))


@pytest.mark.parametrize("g,hkv,seed,m,split", [
    (4, 2, 231, [3, 8, 1, 5, 8], None),       # at most 32 rows: one 32-row tile
    (8, 1, 232, [2, 1, 2, 0, 2], None),       # at most 16 rows: one 16-row tile
    (8, 1, 233, [8, 3, 5, 7, 1], 8),          # 64 rows: two 32-row tiles, 8-block splits
    (4, 2, 234, [30, 12, 1, 25, 9], None),    # 120 rows: four row tiles
    (1, 3, 235, [40, 3, 17, 1, 26], 5),       # g = 1, 40 rows, splits ending inside a wave's blocks
    (2, 2, 236, [16, 4, 0, 1, 12], 3),        # 32 rows, a sequence without query tokens
])
def test_mxfp4(g, hkv, seed, m, split):
    """MX-FP4 caches: the scaled-MFMA multi-token kernel with 16- and 32-row
    tiles, several row tiles per (sequence, kv-head), split merges."""
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=5, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=128,
                                 ctx_range=(60, 700), seed=seed, fmt=1)
    say(f"case: multi-token MX-FP4 g={g} hkv={hkv} seed={seed} m={m} split={split}")
    _run(Case(cfg), np.array(m))


def test_mxfp4_whole_contexts_and_longest_split():
    """MX-FP4: query tokens that are whole contexts (the first row sees one
    key), then 256-block splits of 9000- to 12000-token contexts, where each
    of a work-group's four waves walks 64 blocks (the most one wave-wide id
    load holds)."""
    cfg = workloads.small_config(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(1, 40),
                                 seed=237, fmt=1)
    say("case: multi-token MX-FP4, whole short contexts")
    _run(Case(cfg), np.array([10 ** 6, 10 ** 6, 3, 10 ** 6]))
    os.environ["TQ_SPLIT_BLOCKS"] = "256"
    cfg = workloads.small_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(9000, 12000),
                                 seed=238, fmt=1)
    say("case: multi-token MX-FP4 with 256-block splits")
    _run(Case(cfg), 20)


def test_prefill_from_the_first_token_and_empty_sequences():
    cfg = workloads.small_config(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(30, 300),
                                 seed=208)
    case = Case(cfg)
    m = np.array([10 ** 6, 0, 17, 10 ** 6])     # whole contexts, none, a chunk
    say("case: multi-token prefill of whole contexts with an empty sequence")
    _run(case, m)


def _bf16_of(case, m, split):
    """bf16 output of the same call: must be the RNE rounding of its fp32 output."""
    w, c = case.w, case.cfg
    qbits, q_start = w.multi_queries(m)
    ctx = w.total_lens.astype(np.int32)
    args = (to_dev_bf16(qbits), to_dev_i32(q_start), int(np.max(np.diff(q_start))), case.table_dev, to_dev_i32(ctx),
            int(ctx.max()), c.scale)
    o32 = case.cache.multitoken(*args, out_dtype=torch.float32)
    o16 = case.cache.multitoken(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = workloads.f32_to_bf16_bits(o32.cpu().numpy())
    got = o16.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want), f"split {split}: bf16 output is not the rounded fp32 output"


def test_bf16_output_and_split_invariance():
    cfg = workloads.small_config(batch=3, num_q_heads=16, num_kv_heads=2, head_dim=128, ctx_range=(900, 2000),
                                 seed=209)
    say("case: multi-token split invariance and bf16 output (one split, then 8-block splits)")
    case = Case(cfg)
    a, _ = _run(case, 24)
    _bf16_of(case, 24, None)
    os.environ["TQ_SPLIT_BLOCKS"] = "8"
    b, _ = _run(Case(cfg), 24)
    _bf16_of(case, 24, 8)
    assert np.max(np.abs(a - b)) <= 2e-3 * np.max(np.abs(a))


def test_one_query_token_matches_decode():
    """One query token per sequence through the multi-token path equals the
    decode path up to their one numerical difference: the multi-token kernels
    round the probabilities once to fp16 (at most 2^-11 relative, unbiased),
    the decode kernel carries them as fp16 high + low parts."""
    cfg = workloads.small_config(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(50, 900),
                                 seed=210)
    case = Case(cfg)
    out, q_start = _run(case, 1)
    qbits, _ = case.w.multi_queries(1)
    ctx = case.w.total_lens.astype(np.int32)
    dec = case.cache.decode(to_dev_bf16(qbits), case.table_dev, to_dev_i32(ctx), int(ctx.max()), cfg.scale)
    torch.cuda.synchronize()
    assert row_rel_err(out, dec.cpu().numpy()) <= 1e-3


@pytest.mark.parametrize("name", ["verify", "prefill"])
def test_full_size_sampled(name):
    cfg = workloads.MT_CONFIGS[name]
    m = workloads.MT_QUERY_TOKENS[name]
    case = Case(cfg)
    rng = np.random.default_rng(211)
    seqs = sorted(rng.choice(cfg.batch, size=min(2, cfg.batch), replace=False).tolist())
    qbits, q_start = case.w.multi_queries(m)
    rows = []
    for b in seqs:
        toks = rng.choice(np.arange(int(q_start[b]), int(q_start[b + 1])), size=min(4, m), replace=False)
        rows += [(int(i), int(h)) for i in toks for h in rng.choice(cfg.num_q_heads, size=3, replace=False)]
    say(f"case: multi-token full size {name}: sampled sequences {seqs}, {len(rows)} rows")
    _run(case, m, rows=rows, seqs=seqs)


def test_long_split_walks_more_than_64_blocks_per_wave():
    # 1024-block splits: each wave walks up to ~94 blocks, past the 64 block
    # ids one wave-wide load holds
    os.environ["TQ_SPLIT_BLOCKS"] = "1024"
    cfg = workloads.small_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(9000, 12000),
                                 seed=212)
    say("case: multi-token with 1024-block splits (block ids fetched in chunks of 64 per wave)")
    _run(Case(cfg), 40)


@pytest.mark.parametrize("d,g,hkv,seed,mmax,split", [
    (128, 4, 2, 213, 8, None), (128, 8, 1, 214, 2, 3), (128, 1, 3, 215, 16, None), (128, 2, 2, 216, 16, 5),
    (128, 4, 1, 217, 4, 1), (64, 4, 2, 218, 8, 7), (64, 8, 1, 219, 4, None), (64, 2, 2, 220, 8, 2),
    (128, 1, 2, 224, 32, None), (64, 1, 1, 225, 32, 3),
])
def test_direct_kernel_small_row_counts(d, g, hkv, seed, mmax, split):
    """At most 32 rows per (sequence, kv-head): the direct kernel (16- or
    32-row tiles), ragged query counts (zero included), odd split sizes that
    end splits inside a block pair, and lone last pairs."""
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=5, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                                 ctx_range=(1, 700), seed=seed)
    rng = np.random.default_rng(seed)
    m = rng.integers(0, mmax + 1, size=5)
    m[rng.integers(0, 5)] = mmax
    assert mmax * g <= 32
    say(f"case: multi-token direct d={d} g={g} hkv={hkv} seed={seed} m={m.tolist()} split={split}")
    _run(Case(cfg), m)


def test_direct_kernel_whole_short_contexts_bf16_and_long_splits():
    """Direct kernel: query tokens that are the whole (short) context, so the
    first rows see one key; bf16 output equal to the rounded fp32 output; and
    1024-block splits, where a wave walks more than the 32 block pairs one
    wave-wide id load holds."""
    cfg = workloads.small_config(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(1, 8),
                                 seed=221)
    say("case: multi-token direct, whole short contexts")
    _run(Case(cfg), 10 ** 6)
    cfg = workloads.small_config(batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128, ctx_range=(900, 2000),
                                 seed=222)
    say("case: multi-token direct, bf16 output")
    case = Case(cfg)
    _run(case, 8)
    _bf16_of(case, 8, None)
    os.environ["TQ_SPLIT_BLOCKS"] = "1024"
    cfg = workloads.small_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(9000, 12000),
                                 seed=223)
    say("case: multi-token direct, 1024-block splits (block ids fetched in chunks of 32 pairs per wave)")
    _run(Case(cfg), 8)


@pytest.mark.parametrize("fmt,v_scale,m,seed", [
    (0, 3.0e4, [3, 8, 1], 231),        # scales >= 4096: direct kernel (at most 32 rows)
    (0, 3.0e4, [40, 12, 25], 232),     # and the staged kernel
    (2, 3.0e4, [40, 12, 25], 233),
    (0, 1.0e-6, [3, 8, 1], 234),       # fp16-subnormal scales and minima
    (0, 1.0e-6, [40, 12, 25], 235),
])
def test_value_range_edges(fmt, v_scale, m, seed):
    """Value groups beyond the fp16 range and tiny ones: the dequantized values
    enter the products exactly in both kernels."""
    cfg = workloads.small_config(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(60, 500),
                                 seed=seed, fmt=fmt, v_scale=v_scale)
    say(f"case: multi-token value range fmt={fmt} v_scale={v_scale:g} m={m} seed={seed}")
    _run(Case(cfg), np.array(m))
