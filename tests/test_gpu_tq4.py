"""GPU parity of the TQ4/4 path against the CPU oracle, through the C ABI.

Packed bytes must be identical (codes, scales, layout); decode attention must
be within 2e-3 (max over rows of ||o - o_ref||_inf / ||o_ref||_inf) of the
oracle's exact fp64 attention over the same dequantized cache."""
import os

import numpy as np
import pytest
import torch

import workloads
from gpu_common import TOL, Case, check_case as _check_case, row_rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _split_env():
    saved = {k: os.environ.pop(k, None) for k in ("TQ_SPLIT_BLOCKS",)}
    yield
    for k, v in saved.items():
        os.environ.pop(k, None)
        if v is not None:
            os.environ[k] = v


def test_tiny_config():
    say("case: tiny (1 seq, 1 kv head, g=4, D=64, T=256)")
    _check_case(Case(workloads.CONFIGS["tiny"]))


@pytest.mark.parametrize("d,g,hkv,seed,split", [
    (128, 4, 2, 101, None), (128, 8, 1, 102, None), (128, 1, 3, 103, 4), (128, 2, 2, 104, 8),
    (64, 4, 2, 105, None), (64, 8, 1, 106, 4), (64, 1, 2, 107, None), (64, 2, 1, 108, 12),
])
def test_small_ragged(d, g, hkv, seed, split):
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=5, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d,
                                 ctx_range=(1, 700), seed=seed)
    say(f"case: small ragged d={d} g={g} hkv={hkv} seed={seed} split={split}")
    _check_case(Case(cfg))


def test_edge_lengths_and_zero_context():
    cfg = workloads.small_config(batch=6, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(1, 40), seed=109)
    case = Case(cfg)
    ranges = case.write_ranges()
    case.quantize(ranges)
    op = case.oracle_pool(ranges)
    ctx = np.array([0, 1, 15, 16, 17, 32], np.int32)
    ctx = np.minimum(ctx, case.w.prompt_lens.astype(np.int32))
    say(f"case: edge lengths {ctx.tolist()}")
    out = case.decode(ctx=ctx)
    rows = [(b, h) for b in range(6) for h in range(8)]
    ref = case.oracle_decode(op, rows, ctx=ctx)
    assert np.all(out[ctx == 0] == 0)
    assert row_rel_err(out, ref) <= TOL


def test_split_merge_with_zero_and_short_contexts():
    """Many splits per sequence merged by the merge kernel, mixed with a
    sequence without tokens and one that fits in a single split; repeated
    calls give the same result."""
    cfg = workloads.small_config(batch=6, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(300, 900), seed=114)
    case = Case(cfg)
    ranges = case.write_ranges()
    case.quantize(ranges)
    op = case.oracle_pool(ranges)
    ctx = case.w.prompt_lens.astype(np.int32).copy()
    ctx[1], ctx[4] = 0, 100
    os.environ["TQ_SPLIT_BLOCKS"] = "8"
    say(f"case: split merge, contexts {ctx.tolist()}")
    rows = [(b, h) for b in range(6) for h in range(8)]
    ref = case.oracle_decode(op, rows, ctx=ctx)
    first = None
    for _ in range(3):
        out = case.decode(ctx=ctx)
        assert np.all(out[1] == 0)
        assert row_rel_err(out, ref) <= TOL
        first = out if first is None else first
        assert np.array_equal(out, first)


def test_bf16_output():
    cfg = workloads.small_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(100, 300), seed=110)
    case = Case(cfg)
    case.quantize(case.write_ranges())
    say("case: bf16 output")
    o32 = case.decode()
    o16 = case.decode(out_dtype=torch.bfloat16)
    assert np.max(np.abs(o16 - o32)) <= np.max(np.abs(o32)) * 2 ** -8


def test_unaligned_skipped_and_single_token_slots():
    """Slots that break the four-row fast path, skipped tokens, and appends
    of one token at a time must give the same bytes as the oracle."""
    cfg = workloads.small_config(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=128, ctx_range=(160, 160),
                                 seed=111)
    w = workloads.make(cfg)
    from bit_quantized_kv_amd import Cache
    from gpu_common import to_dev_bf16, to_dev_i32
    from oracle import paged
    k, v = w.sequence_kv(0)
    rng = np.random.default_rng(5)
    slots = rng.permutation(w.num_blocks * 16)[:160].astype(np.int32)
    slots[rng.choice(160, 20, replace=False)] = -1
    cache = Cache(0, 128, 2, w.num_blocks)
    say("case: permuted slots with skips, then one-token appends")
    cache.quantize_append(to_dev_bf16(k[:100]), to_dev_bf16(v[:100]), to_dev_i32(slots[:100]))
    for i in range(100, 160):
        cache.quantize_append(to_dev_bf16(k[i:i + 1]), to_dev_bf16(v[i:i + 1]), to_dev_i32(slots[i:i + 1]))
    torch.cuda.synchronize()
    gpu = cache.pool.cpu().numpy().reshape(w.num_blocks, 2, -1)
    op = paged.PagedPool(0, w.num_blocks, 2, 128)
    op.append(workloads.bf16_bits_to_f32(k), workloads.bf16_bits_to_f32(v), slots)
    assert np.array_equal(gpu, op.pool)


@pytest.fixture
def _loop_env():
    saved = {k: os.environ.pop(k, None) for k in ("TQ_QUANT_LOOP", "TQ_ITEM_WINDOW")}
    yield
    for k, v in saved.items():
        os.environ.pop(k, None)
        if v is not None:
            os.environ[k] = v


@pytest.mark.parametrize("loop", ["static", "balanced", "balanced-pairs"])
@pytest.mark.parametrize("fmt,d,hkv,seed", [(0, 128, 3, 141), (0, 64, 2, 142), (2, 128, 2, 143), (2, 64, 3, 144)])
def test_both_quantize_loops(_loop_env, loop, fmt, d, hkv, seed):
    """Every work distribution of the quantize kernel (fixed shares per
    work-group, or per-compute-unit ranges handed out to waves by a counter,
    one task or a pair at a time) writes the oracle's bytes, for TQ4/4 and
    TQ4/2 at both head sizes."""
    os.environ["TQ_QUANT_LOOP"] = loop
    # about 15000 tokens: the balanced loop's 256 work-groups take 3 to 30
    # tasks each (the counter is asked in some of them; the long launches
    # below make every wave ask it)
    cfg = workloads.small_config(batch=6, num_q_heads=4 * hkv, num_kv_heads=hkv, head_dim=d, ctx_range=(1500, 3000),
                                 seed=seed, fmt=fmt)
    say(f"case: quantize loop {loop}, format {fmt}, d={d}, hkv={hkv}, seed={seed}")
    _check_case(Case(cfg))


@pytest.mark.parametrize("loop,fmt,d,hkv,seed", [("balanced", 0, 128, 2, 145), ("balanced-pairs", 0, 128, 2, 146),
                                                 ("balanced-pairs", 2, 64, 4, 147), ("balanced-pairs", 1, 128, 2, 148)])
def test_balanced_loop_hands_out_from_the_counter(_loop_env, loop, fmt, d, hkv, seed):
    """A launch long enough that every work-group of the balanced loop takes
    several times the 16 (one by one) or 32 (pairs) tasks its waves start
    with, so that tasks and pairs of tasks come from the LDS counter; the
    records match the oracle's byte for byte (TQ4/4, TQ4/2 and MX-FP4)."""
    os.environ["TQ_QUANT_LOOP"] = loop
    cfg = workloads.small_config(batch=8, num_q_heads=4 * hkv, num_kv_heads=hkv, head_dim=d, ctx_range=(12000, 16000),
                                 seed=seed, fmt=fmt)
    case = Case(cfg)
    tpw = 8 if d == 128 else 16
    tasks_per_wg = int(case.w.total_lens.sum()) // tpw * hkv / 256
    say(f"case: quantize loop {loop}, format {fmt}, d={d}, hkv={hkv}, seed={seed}, "
        f"about {tasks_per_wg:.0f} tasks per work-group")
    assert tasks_per_wg > 3 * 32
    ranges = case.write_ranges()
    case.quantize(ranges)
    op = case.oracle_pool(ranges)
    gpu = case.pool_np()
    bad = np.nonzero(np.any(gpu != op.pool, axis=(1, 2)))[0]
    assert bad.size == 0, f"{bad.size} blocks differ from the oracle's, first {bad[:4]}"


def _scattered_launch(rng, num_blocks, n_seq):
    """Slots of one launch: sequences that start at arbitrary rows of fresh
    blocks and run 1 to 300 rows (so the launch's token order cuts them
    anywhere), a stretch of single rows at scattered slots, and skipped
    tokens (-1) sprinkled over both."""
    parts, blk = [], 0
    for _ in range(n_seq):
        off, length = int(rng.integers(0, 16)), int(rng.integers(1, 301))
        parts.append(np.arange(blk * 16 + off, blk * 16 + off + length))
        blk += (off + length + 15) // 16
    used = np.concatenate(parts)
    free = np.setdiff1d(np.arange(num_blocks * 16), np.arange(blk * 16))
    scattered = rng.permutation(free)[:600]
    slots = np.concatenate(parts[:n_seq // 2] + [scattered] + parts[n_seq // 2:]).astype(np.int32)
    slots[rng.choice(slots.size, slots.size // 50, replace=False)] = -1
    assert used.max() < num_blocks * 16
    return slots


@pytest.mark.parametrize("fmt,d,window,seed", [(0, 128, 97, 151), (0, 64, 61, 152), (2, 128, 8192, 153),
                                               (2, 64, 200, 154), (1, 128, 113, 155)])
def test_balanced_loop_items_and_windows(_loop_env, fmt, d, window, seed):
    """The balanced loop cuts each work-group's token range into items (runs of
    rows inside one aligned span of a block, placed on the lanes of their rows)
    and lists them in windows.  Sequences starting at any row, scattered single
    rows and skipped tokens, listed in windows of a few dozen tokens (several
    per work-group) or in one, give the oracle's bytes for TQ4/4, TQ4/2 and
    MX-FP4."""
    from bit_quantized_kv_amd import Cache
    from gpu_common import to_dev_bf16, to_dev_i32
    from oracle import paged
    os.environ["TQ_QUANT_LOOP"] = "balanced"
    os.environ["TQ_ITEM_WINDOW"] = str(window)
    rng = np.random.default_rng(seed)
    hkv, num_blocks = 2, 2048
    slots = _scattered_launch(rng, num_blocks, 120)
    n = slots.size
    kf = rng.standard_normal((n, hkv, d)).astype(np.float32) * np.float32(2.0)
    vf = rng.standard_normal((n, hkv, d)).astype(np.float32)
    kb, vb = workloads.f32_to_bf16_bits(kf), workloads.f32_to_bf16_bits(vf)
    say(f"case: balanced-loop items, format {fmt}, d={d}, window {window}, seed {seed}, {n} tokens")
    cache = Cache(fmt, d, hkv, num_blocks)
    cache.quantize_append(to_dev_bf16(kb), to_dev_bf16(vb), to_dev_i32(slots))
    torch.cuda.synchronize()
    gpu = cache.pool.cpu().numpy().reshape(num_blocks, hkv, -1)
    op = paged.PagedPool(fmt, num_blocks, hkv, d)
    op.append(workloads.bf16_bits_to_f32(kb), workloads.bf16_bits_to_f32(vb), slots)
    bad = np.nonzero(np.any(gpu != op.pool, axis=(1, 2)))[0]
    assert bad.size == 0, f"{bad.size} blocks differ from the oracle's, first {bad[:4]}"


@pytest.mark.parametrize("d,window,seed", [(64, 8192, 161), (128, 1100, 162)])
def test_balanced_loop_listing_rounds(_loop_env, d, window, seed):
    """Work-group ranges of more than 1024 tokens are listed in several rounds
    of the work-group's threads, and items (runs of rows in one span of a
    block) start in one round and end in the next.  About 300000 tokens of
    sequences that start at any row of a block: the records match the
    oracle's byte for byte (regression: the round-crossing items once got the
    wrong last row)."""
    from bit_quantized_kv_amd import Cache
    from gpu_common import to_dev_bf16, to_dev_i32
    from oracle import paged
    os.environ["TQ_QUANT_LOOP"] = "balanced"
    os.environ["TQ_ITEM_WINDOW"] = str(window)
    rng = np.random.default_rng(seed)
    parts, blk = [], 0
    while sum(p.size for p in parts) < 300000:
        off, length = int(rng.integers(0, 16)), int(rng.integers(1, 2000))
        parts.append(np.arange(blk * 16 + off, blk * 16 + off + length))
        blk += (off + length + 15) // 16
    slots = np.concatenate(parts).astype(np.int32)
    n, num_blocks = slots.size, blk
    assert n // 256 > 1024  # every work-group lists its range in two rounds or more
    kf = rng.standard_normal((n, 1, d)).astype(np.float32)
    vf = rng.standard_normal((n, 1, d)).astype(np.float32) * np.float32(0.5)
    kb, vb = workloads.f32_to_bf16_bits(kf), workloads.f32_to_bf16_bits(vf)
    say(f"case: balanced-loop listing rounds, d={d}, window {window}, seed {seed}, {n} tokens")
    cache = Cache(0, d, 1, num_blocks)
    cache.quantize_append(to_dev_bf16(kb), to_dev_bf16(vb), to_dev_i32(slots))
    torch.cuda.synchronize()
    gpu = cache.pool.cpu().numpy().reshape(num_blocks, 1, -1)
    op = paged.PagedPool(0, num_blocks, 1, d)
    op.append(workloads.bf16_bits_to_f32(kb), workloads.bf16_bits_to_f32(vb), slots)
    bad = np.nonzero(np.any(gpu != op.pool, axis=(1, 2)))[0]
    assert bad.size == 0, f"{bad.size} blocks differ from the oracle's, first {bad[:4]}"


@pytest.mark.parametrize("fmt,d,hkv,n,seed", [(0, 128, 1, 1, 171), (0, 64, 8, 5, 172), (2, 128, 8, 300, 173),
                                               (1, 128, 3, 77, 174)])
def test_balanced_loop_short_launches(_loop_env, fmt, d, hkv, n, seed):
    """The balanced loop forced on launches shorter than its grid: most
    work-groups get an empty token range, the others one or a few items;
    slots are scattered (every row its own item) with skips.  The records
    match the oracle's byte for byte."""
    from bit_quantized_kv_amd import Cache
    from gpu_common import to_dev_bf16, to_dev_i32
    from oracle import paged
    os.environ["TQ_QUANT_LOOP"] = "balanced"
    rng = np.random.default_rng(seed)
    num_blocks = 64
    slots = rng.permutation(num_blocks * 16)[:n].astype(np.int32)
    if n > 2:
        slots[rng.choice(n, max(1, n // 10), replace=False)] = -1
    kf = rng.standard_normal((n, hkv, d)).astype(np.float32)
    vf = rng.standard_normal((n, hkv, d)).astype(np.float32)
    kb, vb = workloads.f32_to_bf16_bits(kf), workloads.f32_to_bf16_bits(vf)
    say(f"case: balanced loop, short launch of {n} tokens, format {fmt}, d={d}, hkv={hkv}, seed {seed}")
    cache = Cache(fmt, d, hkv, num_blocks)
    cache.quantize_append(to_dev_bf16(kb), to_dev_bf16(vb), to_dev_i32(slots))
    torch.cuda.synchronize()
    gpu = cache.pool.cpu().numpy().reshape(num_blocks, hkv, -1)
    op = paged.PagedPool(fmt, num_blocks, hkv, d)
    op.append(workloads.bf16_bits_to_f32(kb), workloads.bf16_bits_to_f32(vb), slots)
    assert np.array_equal(gpu, op.pool)


def test_pool_beyond_4_gib():
    """A 4.7 GB pool (10^6 blocks x 2 kv-heads x 2336 B): records past byte
    2^32 are written and read through 64-bit offsets.  One sequence lives on
    the pool's first blocks, one on its last; their records, decode and
    multi-token attention match the oracle, which holds the same blocks in a
    compact pool (block b * 19 + j for the GPU's block j of sequence b)."""
    from bit_quantized_kv_amd import Cache
    from gpu_common import to_dev_bf16, to_dev_i32
    from oracle import attention, paged
    nblk, hkv, d, g, T = 1_000_000, 2, 128, 4, 300
    nb = (T + 15) // 16
    cfg = workloads.small_config(batch=2, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, ctx_range=(T, T),
                                 seed=131)
    w = workloads.make(cfg)
    rng = np.random.default_rng(131)
    ids = np.stack([rng.permutation(nb), nblk - 1 - rng.permutation(nb)]).astype(np.int32)
    compact = np.arange(2 * nb, dtype=np.int32).reshape(2, nb)
    t = np.arange(T)
    kb = np.concatenate([w.sequence_kv(b)[0][:T] for b in range(2)])
    vb = np.concatenate([w.sequence_kv(b)[1][:T] for b in range(2)])
    slots = np.concatenate([ids[b][t // 16] * 16 + t % 16 for b in range(2)]).astype(np.int32)
    oslots = np.concatenate([compact[b][t // 16] * 16 + t % 16 for b in range(2)]).astype(np.int32)
    cache = Cache(0, d, hkv, nblk)
    assert cache.pool.numel() > 2 ** 32
    say(f"case: pool of {cache.pool.numel() / 1e9:.2f} GB, blocks {ids[1].min()}..{ids[1].max()} at its end")
    cache.quantize_append(to_dev_bf16(kb), to_dev_bf16(vb), to_dev_i32(slots))
    sel = torch.from_numpy(ids.ravel().astype(np.int64)).cuda()
    gpu = cache.pool.view(nblk, hkv, -1)[sel].cpu().numpy()
    op = paged.PagedPool(0, 2 * nb, hkv, d)
    op.append(workloads.bf16_bits_to_f32(kb), workloads.bf16_bits_to_f32(vb), oslots)
    assert np.array_equal(gpu, op.pool), "records past 4 GiB differ from the oracle's"
    ctx = np.array([T, T], np.int32)
    qbits = w.query_bits(0)
    out = cache.decode(to_dev_bf16(qbits), to_dev_i32(ids), to_dev_i32(ctx), T, cfg.scale).cpu().numpy()
    ref = attention.decode(op, workloads.bf16_bits_to_f32(qbits), compact, ctx, cfg.scale)
    err = row_rel_err(out.reshape(-1, d), ref.reshape(-1, d))
    say(f"  decode: max rel err {err:.2e}")
    assert err <= TOL
    mq, q_start = w.multi_queries(8)
    mt = cache.multitoken(to_dev_bf16(mq), to_dev_i32(q_start), 8, to_dev_i32(ids), to_dev_i32(ctx), T,
                          cfg.scale).float().cpu().numpy()
    mref = attention.multi_token(op, workloads.bf16_bits_to_f32(mq), q_start, compact, ctx, cfg.scale)
    err = row_rel_err(mt.reshape(-1, d), mref.reshape(-1, d))
    say(f"  multi-token: max rel err {err:.2e}")
    assert err <= TOL


def test_custom_key_table():
    table = list(np.linspace(-2.5, 2.5, 16))
    cfg = workloads.small_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(50, 400), seed=112)
    say("case: uniform custom key table")
    case = Case(cfg, key_table=table)
    _check_case(case)


def test_determinism_and_split_invariance():
    cfg = workloads.small_config(batch=3, num_q_heads=16, num_kv_heads=2, head_dim=128, ctx_range=(900, 2000),
                                 seed=113)
    case = Case(cfg)
    case.quantize(case.write_ranges())
    a = case.pool_np().copy()
    case.quantize(case.write_ranges())
    assert np.array_equal(a, case.pool_np())
    say("case: split invariance 4 / 16 / 64 blocks")
    outs = []
    for sb in ("4", "16", "64"):
        os.environ["TQ_SPLIT_BLOCKS"] = sb
        outs.append(case.decode())
    assert row_rel_err(outs[0], outs[1]) <= 2e-4 and row_rel_err(outs[0], outs[2]) <= 2e-4


def test_full_llama8b():
    say("case: llama8b layer (B=1, 32/8, D=128, T=32768), full pool and all rows")
    _check_case(Case(workloads.CONFIGS["llama8b"]))


def test_full_agentic_sampled():
    say("case: agentic (B=32, shared prefixes), sampled sequences")
    _check_case(Case(workloads.CONFIGS["agentic"]), seqs=[0, 9, 15, 16, 31])


def test_full_longprefix_sampled_steps():
    cfg = workloads.CONFIGS["longprefix"]
    case = Case(cfg)
    w = case.w
    say("case: longprefix quantize 8 x 25600 tokens, then 64 one-token appends + decodes")
    case.quantize(case.write_ranges())
    seqs = [0, 5]
    from gpu_common import to_dev_bf16, to_dev_i32
    kv = [w.sequence_kv(b) for b in range(cfg.batch)]
    checks = (0, 31, 63)
    gpu_outs = {}
    for step in range(cfg.decode_steps):
        t = int(w.prompt_lens[0]) + step
        k = np.concatenate([kv[b][0][t:t + 1] for b in range(cfg.batch)])
        v = np.concatenate([kv[b][1][t:t + 1] for b in range(cfg.batch)])
        s = np.concatenate([w.slots(b, t, t + 1) for b in range(cfg.batch)])
        case.cache.quantize_append(to_dev_bf16(k), to_dev_bf16(v), to_dev_i32(s))
        if step in checks:
            gpu_outs[step] = case.decode(step)
    say("  steps done; building the oracle for sampled sequences")
    op = case.oracle_pool([(b, 0, int(w.total_lens[b])) for b in seqs])
    gpu = case.pool_np()
    blocks = case.blocks_of(seqs)
    assert np.array_equal(gpu[blocks], op.pool[blocks])
    for step in checks:
        rows = [(b, h) for b in seqs for h in range(0, cfg.num_q_heads, 7)]
        ref = case.oracle_decode(op, rows, step)
        err = row_rel_err(np.array([gpu_outs[step][b, h] for b, h in rows]), np.array([ref[b, h] for b, h in rows]))
        say(f"  step {step}: max rel err {err:.2e}")
        assert err <= TOL


def test_longest_split_per_wave():
    """512-block splits: a wave of the decode kernel walks 64 blocks, the most
    one wave-wide block-id load holds; contexts of 9000 to 12000 tokens."""
    os.environ["TQ_SPLIT_BLOCKS"] = "512"
    cfg = workloads.small_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(9000, 12000),
                                 seed=116)
    say("case: decode with 512-block splits (64 blocks per wave)")
    _check_case(Case(cfg))
