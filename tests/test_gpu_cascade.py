"""GPU parity of shared-prefix (cascade) decode against the CPU oracle's
decode, through the C ABI: the same rows as tq_decode_attention, within 2e-3
(max over rows of ||o - o_ref||_inf / ||o_ref||_inf), over a byte-identical
cache; the GPU's own plain decode agrees to well inside that."""
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


def _run(case, groups, seqs=None, ctx=None, rows=None, max_members=None):
    c, w = case.cfg, case.w
    ranges = case.write_ranges()
    case.quantize(ranges)
    seqs = list(range(c.batch)) if seqs is None else seqs
    gpu_pool = case.pool_np()
    writer = w.prefix_writer()
    op = case.oracle_pool([r for r in ranges if r[0] in seqs or r[0] == writer])
    blocks = case.blocks_of(seqs)
    assert np.array_equal(gpu_pool[blocks], op.pool[blocks]), "cache records differ from the oracle's"
    ctx = w.context_lens_at(0) if ctx is None else np.asarray(ctx, np.int32)
    q = to_dev_bf16(w.query_bits(0))
    from bit_quantized_kv_amd import CascadeGroups
    out = case.cache.cascade_decode(q, case.table_dev, to_dev_i32(ctx), int(ctx.max()), c.scale,
                                    CascadeGroups(c.batch, groups, max_members=max_members))
    plain = case.cache.decode(q, case.table_dev, to_dev_i32(ctx), int(ctx.max()), c.scale)
    torch.cuda.synchronize()
    out, plain = out.cpu().numpy(), plain.cpu().numpy()
    rows = rows if rows is not None else [(b, h) for b in seqs for h in range(c.num_q_heads)]
    ref = attention.decode(op, workloads.bf16_bits_to_f32(w.query_bits(0)), w.block_table, ctx, c.scale, rows=rows)
    ora = attention.cascade_decode(op, workloads.bf16_bits_to_f32(w.query_bits(0)), w.block_table, ctx, c.scale,
                                   groups, rows=rows[:8])
    assert row_rel_err(np.array([ora[b, h] for b, h in rows[:8]]), np.array([ref[b, h] for b, h in rows[:8]])) < 1e-10
    err = row_rel_err(np.array([out[b, h] for b, h in rows]), np.array([ref[b, h] for b, h in rows]))
    dif = row_rel_err(out, plain)
    say(f"  {c.name}: {len(rows)} rows, max rel err {err:.2e} (vs plain GPU decode {dif:.2e})")
    assert err <= TOL
    assert dif <= 1e-3
    return out


@pytest.mark.parametrize("d,g,hkv,seed,split", [
    (128, 4, 2, 301, None), (128, 8, 1, 302, 4), (128, 1, 2, 303, 8), (64, 2, 2, 304, None), (64, 4, 1, 305, 4),
])
def test_small_groups(d, g, hkv, seed, split):
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=6, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, ctx_range=(170, 600),
                                 shared_seqs=3, shared_tokens=160, seed=seed)
    say(f"case: cascade d={d} g={g} hkv={hkv} seed={seed} split={split}: sequences 0-2 share 10 blocks, "
        f"nested as 0-3 for all and 4-9 for sequences 0 and 2; sequence 4 alone in a 3-block group")
    _run(Case(cfg), [([0, 1, 2], 0, 4), ([0, 2], 4, 10), ([4], 0, 3)])


@pytest.mark.parametrize("d,g,hkv,seed,split", [(128, 4, 2, 311, None), (64, 8, 1, 312, 4)])
def test_two_bit_values(d, g, hkv, seed, split):
    """TQ4/2 caches with nested groups: at g = 4 every group takes the direct
    kernel; at g = 8 the 6-sequence group's 48 rows take the staged one."""
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=7, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, ctx_range=(200, 600),
                                 shared_seqs=6, shared_tokens=160, seed=seed, fmt=2)
    say(f"case: cascade TQ4/2 d={d} g={g} hkv={hkv} seed={seed} split={split}")
    _run(Case(cfg), [([0, 1, 2, 3, 4, 5], 0, 4), ([0, 2, 4], 4, 10), ([6], 0, 3)])


@pytest.mark.parametrize("g,hkv,seed,split", [(4, 2, 321, None), (8, 1, 322, 4), (1, 2, 323, 8)])
def test_mxfp4(g, hkv, seed, split):
    """MX-FP4 caches with nested groups: the own-token pass on the MX-FP4
    decode kernel, the shared blocks on its multi-token kernel in prefix mode
    (at g = 8 the 6-sequence group's 48 rows take two 32-row tiles)."""
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=7, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=128,
                                 ctx_range=(200, 600), shared_seqs=6, shared_tokens=160, seed=seed, fmt=1)
    say(f"case: cascade MX-FP4 g={g} hkv={hkv} seed={seed} split={split}")
    _run(Case(cfg), [([0, 1, 2, 3, 4, 5], 0, 4), ([0, 2, 4], 4, 10), ([6], 0, 3)])


def test_context_ending_at_the_prefix_and_no_groups():
    cfg = workloads.small_config(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(200, 400),
                                 shared_seqs=2, shared_tokens=192, seed=306)
    case = Case(cfg)
    ctx = case.w.context_lens_at(0).copy()
    ctx[0] = 192                          # nothing of its own after the 12 shared blocks
    say("case: cascade, a member whose context is exactly the shared prefix")
    _run(case, [([0, 1], 0, 12)], ctx=ctx)
    say("case: cascade with no groups (plain decode through the cascade path)")
    _run(Case(cfg), [])


@pytest.mark.parametrize("max_members", [None, 3])
def test_large_group_staged_and_cut(max_members):
    """A group of 6 sequences at g = 8 (48 rows: the staged kernel), and the
    same group cut into groups of at most 3 members (24 rows: the direct
    kernel), with a nested group below it."""
    cfg = workloads.small_config(batch=7, num_q_heads=8, num_kv_heads=1, head_dim=128, ctx_range=(200, 500),
                                 shared_seqs=6, shared_tokens=160, seed=307)
    say(f"case: cascade, a 6-sequence group over 10 shared blocks, max_members={max_members}")
    _run(Case(cfg), [([0, 1, 2, 3, 4, 5], 0, 6), ([1, 3, 5], 6, 10)], max_members=max_members)


@pytest.mark.parametrize("max_members", [None, 8])
def test_full_agentic_sampled(max_members):
    """The agentic workload's nested groups as they are (16 sharers: 64 rows,
    the staged kernel) and cut into 8-sequence groups (32 rows, the direct
    kernel)."""
    cfg = workloads.CONFIGS["agentic"]
    case = Case(cfg)
    groups = case.w.shared_block_groups()
    seqs = [0, 6, 9, 15, 16, 31]
    say(f"case: cascade agentic: {len(groups)} nested groups of shared blocks, max_members={max_members}; "
        f"sampled sequences {seqs}")
    _run(case, groups, seqs=seqs, max_members=max_members)


def test_shared_range_longer_than_the_block_id_table_is_refused():
    """A group's shared range is at most 4096 blocks (a work-group stages its
    range's block ids in LDS); the host refuses longer ones before any launch,
    and accepts exactly 4096."""
    from bit_quantized_kv_amd import Cache
    from bit_quantized_kv_amd.binding import TqError, tq_cascade_workspace_bytes
    cache = Cache(0, 128, 2, 16)
    say("case: cascade workspace query with 4096 and 4097 shared blocks")
    assert tq_cascade_workspace_bytes(cache.handle, 2, 8, 16 * 4097, 1, 2, 4096, 1) > 0
    with pytest.raises(TqError):
        tq_cascade_workspace_bytes(cache.handle, 2, 8, 16 * 4097, 1, 2, 4097, 1)


def test_mxfp4_shared_range_longer_than_one_work_group_is_refused():
    """An MX-FP4 group's shared range is at most 256 blocks (its work-group's
    four waves hold 64 block ids each); the host refuses longer ones before
    any launch, and accepts exactly 256."""
    from bit_quantized_kv_amd import Cache
    from bit_quantized_kv_amd.binding import TqError, tq_cascade_workspace_bytes
    cache = Cache(1, 128, 2, 16)
    say("case: MX-FP4 cascade workspace query with 256 and 257 shared blocks")
    assert tq_cascade_workspace_bytes(cache.handle, 2, 8, 16 * 257, 1, 2, 256, 1) > 0
    with pytest.raises(TqError):
        tq_cascade_workspace_bytes(cache.handle, 2, 8, 16 * 257, 1, 2, 257, 1)
