"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, build the oracle's side from the same inputs."""
import os
import sys

import numpy as np
import torch

import workloads
from oracle import attention, paged

TOL = 2e-3   # max over rows of ||o - o_ref||_inf / ||o_ref||_inf


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def row_rel_err(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(out - ref).max(-1)
    den = np.abs(ref).max(-1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1), num)))


class Case:
    """One workload on the GPU and (for chosen sequences) in the oracle."""

    def __init__(self, cfg, key_table=None):
        from bit_quantized_kv_amd import Cache
        self.w = workloads.make(cfg)
        self.cfg = self.w.cfg
        c = self.cfg
        self.cache = Cache(c.fmt, c.head_dim, c.num_kv_heads, self.w.num_blocks, key_table=key_table)
        self.key_table = key_table
        self.table_dev = to_dev_i32(self.w.block_table)

    def write_ranges(self, lens=None):
        """Token ranges that write every cached token once (see workloads)."""
        return self.w.write_plan(lens)

    def quantize(self, ranges, chunk_tokens=1 << 18):
        """One quantize call per chunk of concatenated token ranges."""
        ks, vs, ss, n = [], [], [], 0
        for b, t0, t1 in ranges:
            k, v = self.w.sequence_kv(b)
            ks.append(k[t0:t1])
            vs.append(v[t0:t1])
            ss.append(self.w.slots(b, t0, t1))
            n += t1 - t0
            if n >= chunk_tokens:
                self._q(ks, vs, ss)
                ks, vs, ss, n = [], [], [], 0
        if ks:
            self._q(ks, vs, ss)

    def _q(self, ks, vs, ss):
        k = to_dev_bf16(np.concatenate(ks))
        v = to_dev_bf16(np.concatenate(vs))
        s = to_dev_i32(np.concatenate(ss))
        self.cache.quantize_append(k, v, s)

    def pool_np(self):
        torch.cuda.synchronize()
        rec = self.cache.record_bytes
        return self.cache.pool.cpu().numpy().reshape(self.w.num_blocks, self.cfg.num_kv_heads, rec)

    def oracle_pool(self, ranges):
        c = self.cfg
        tab = None if self.key_table is None else np.asarray(self.key_table, np.float32).astype(np.float16)
        op = paged.PagedPool(c.fmt, self.w.num_blocks, c.num_kv_heads, c.head_dim, tab)
        for b, t0, t1 in ranges:
            k, v = self.w.sequence_kv(b)
            op.append(workloads.bf16_bits_to_f32(k[t0:t1]), workloads.bf16_bits_to_f32(v[t0:t1]),
                      self.w.slots(b, t0, t1))
        return op

    def blocks_of(self, seqs, lens=None):
        ids = []
        for b in seqs:
            n = -(-int((lens if lens is not None else self.w.total_lens)[b]) // 16)
            ids.extend(self.w.block_table[b, :n].tolist())
        return np.unique(np.array(ids, dtype=np.int64))

    def decode(self, step=0, ctx=None, out_dtype=torch.float32):
        c = self.cfg
        q = to_dev_bf16(self.w.query_bits(step))
        ctx = self.w.context_lens_at(step) if ctx is None else np.asarray(ctx, np.int32)
        out = self.cache.decode(q, self.table_dev, to_dev_i32(ctx), int(max(1, ctx.max())), c.scale,
                                out_dtype=out_dtype)
        torch.cuda.synchronize()
        return out.float().cpu().numpy()

    def oracle_decode(self, opool, rows, step=0, ctx=None):
        q = workloads.bf16_bits_to_f32(self.w.query_bits(step))
        ctx = self.w.context_lens_at(step) if ctx is None else np.asarray(ctx, np.int32)
        return attention.decode(opool, q, self.w.block_table, ctx, self.cfg.scale, rows=rows)


def describe_record_diff(gpu_rec, ora_rec, d, fmt=0):
    """Text naming the sections, token rows and values of differing bytes."""
    from oracle import layout
    idx = np.nonzero(gpu_rec != ora_rec)[0]
    sec = {0: layout.tq4_sections, 1: layout.mxfp4_sections, 2: layout.tq4v2_sections}[fmt](d)
    names = sorted(((v, k) for k, v in sec.items() if k != "end"))
    out = []
    for i in idx[:24]:
        name = [k for v, k in names if v <= i][-1]
        out.append(f"{name}+{i - sec[name]}: gpu {gpu_rec[i]:#04x} oracle {ora_rec[i]:#04x}")
    return f"{len(idx)} bytes differ: " + "; ".join(out)


def check_case(case, seqs=None, rows=None, step=0):
    c = case.cfg
    seqs = list(range(c.batch)) if seqs is None else seqs
    ranges = case.write_ranges()
    case.quantize(ranges)
    gpu = case.pool_np()
    writer = case.w.prefix_writer()
    op = case.oracle_pool([r for r in ranges if r[0] in seqs or r[0] == writer])
    blocks = case.blocks_of(seqs)
    mism = np.nonzero(np.any(gpu[blocks] != op.pool[blocks], axis=-1))
    if mism[0].size:
        bi, hi = blocks[mism[0][0]], mism[1][0]
        rows_of = [(b, t) for b in range(c.batch) for t in range(int(case.w.total_lens[b]))
                   if case.w.block_table[b, t // 16] == bi]
        msg = describe_record_diff(gpu[bi, hi], op.pool[bi, hi], c.head_dim, c.fmt)
        raise AssertionError(f"{mism[0].size} records differ; block {bi} head {hi} holds tokens "
                             f"{rows_of[:3]}..{rows_of[-3:]}: {msg}")
    out = case.decode(step)
    rows = rows if rows is not None else [(b, h) for b in seqs for h in range(c.num_q_heads)]
    ref = case.oracle_decode(op, rows, step)
    err = row_rel_err(np.array([out[b, h] for b, h in rows]), np.array([ref[b, h] for b, h in rows]))
    say(f"  {c.name}: {len(blocks)} blocks byte-identical, {len(rows)} rows, max rel err {err:.2e}")
    assert err <= TOL
    return out, ref
