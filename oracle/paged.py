"""Paged cache model: slot mapping on write, block table on read.

Test infrastructure only (see ``oracle/__init__``).

[ST] (first body paragraph after the summary) stores KV in vLLM paged blocks of
16 tokens; [TQ-AMD] spec table and section 1, and [UQ] "這篇論文在解什麼痛點",
describe sessions that reuse the same prefix blocks.  Readings (vLLM style):

* write: token n goes to slot s = slot_mapping[n], i.e. block s // 16,
  row s % 16 of every kv-head's record in that block; s < 0 skips the token;
* read: token t of sequence b lives in block block_table[b, t // 16], row
  t % 16; several sequences may name the same block (shared prefixes);
* a block row that was never written stays as the pool was initialised.

Pinned by tests/test_oracle_attention.py (identity vs permuted block tables,
shared blocks, skipped slots).
"""
import numpy as np

from . import layout, mxfp4, tq4

BLOCK = layout.BLOCK
FORMAT_TQ4 = 0
FORMAT_MXFP4 = 1
FORMAT_TQ4V2 = 2     # 4-bit keys, 2-bit values


class PagedPool:
    def __init__(self, fmt, num_blocks, num_kv_heads, head_dim, key_table_f16=None):
        self.fmt = fmt
        self.num_blocks = num_blocks
        self.hkv = num_kv_heads
        self.d = head_dim
        if fmt in (FORMAT_TQ4, FORMAT_TQ4V2):
            self.rec_bytes = (layout.tq4_record_bytes(head_dim) if fmt == FORMAT_TQ4
                              else layout.tq4v2_record_bytes(head_dim))
            if key_table_f16 is None:
                from .lloyd_max import default_key_table_f16
                key_table_f16 = default_key_table_f16()
            self.table = np.asarray(key_table_f16, dtype=np.float16)
        elif fmt == FORMAT_MXFP4:
            self.rec_bytes = layout.mxfp4_record_bytes(head_dim)
            self.table = None
        else:
            raise ValueError("unknown format")
        self.pool = np.zeros((num_blocks, num_kv_heads, self.rec_bytes), dtype=np.uint8)

    def append(self, k, v, slot_mapping):
        """Encode rows k, v [N, Hkv, D] (fp32 holding bf16 values) into their
        slots.  Duplicate slots in one call: the later token wins."""
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        slots = np.asarray(slot_mapping, dtype=np.int64)
        keep = slots >= 0
        if not keep.any():
            return
        k, v, slots = k[keep], v[keep], slots[keep]
        blk, row = slots // BLOCK, slots % BLOCK
        if np.any(blk >= self.num_blocks):
            raise IndexError("slot outside the pool")
        if self.fmt == FORMAT_TQ4:
            enc = tq4.encode_rows(k, v, self.table)
        elif self.fmt == FORMAT_TQ4V2:
            enc = tq4.encode_rows(k, v, self.table, vlevels=3)
        else:
            enc = mxfp4.encode_rows(k, v)
        # a repeated slot keeps the later token
        _, last = np.unique(slots[::-1], return_index=True)
        sel = np.sort(np.arange(len(slots))[::-1][last])
        flat = self.pool.reshape(-1)
        for h in range(self.hkv):
            base = (blk[sel] * self.hkv + h) * self.rec_bytes
            if self.fmt in (FORMAT_TQ4, FORMAT_TQ4V2):
                write = layout.tq4_write_rows if self.fmt == FORMAT_TQ4 else layout.tq4v2_write_rows
                write(flat, base, row[sel], self.d, enc["kcode"][sel, h], enc["kscale"][sel, h],
                      enc["vcode"][sel, h], enc["vscale"][sel, h], enc["vmin"][sel, h])
            else:
                layout.mxfp4_write_rows(flat, base, row[sel], self.d, enc["kcode"][sel, h], enc["kexp"][sel, h],
                                        enc["vcode"][sel, h], enc["vexp"][sel, h])

    def dequantize_blocks(self, ids):
        """Every row of the records of blocks ``ids`` for every kv-head,
        dequantized as the codecs define it, in fp32: (k_hat_rot, v_hat), each
        [len(ids), Hkv, 16, D] ([TQ-AMD] section 2: k_hat = c[code] * s, v_hat
        = fp32(code * sc + mn); [UQ] "方法怎麼做，白話講": e2m1 * 2^X).  Keys stay
        in the rotated domain."""
        ids = np.asarray(ids, dtype=np.int64)
        recs = self.pool[ids].reshape(-1, self.rec_bytes)
        shape = (len(ids), self.hkv, BLOCK, self.d)
        if self.fmt in (FORMAT_TQ4, FORMAT_TQ4V2):
            sec = (layout.tq4_read_block if self.fmt == FORMAT_TQ4 else layout.tq4v2_read_block)(recs, self.d)
            k = tq4.key_dequant_rot(sec["kcode"], sec["kscale"], self.table)
            v = tq4.value_dequant(sec["vcode"], sec["vscale"], sec["vmin"])
        else:
            sec = layout.mxfp4_read_block(recs, self.d)
            k = mxfp4.mx_decode(sec["kcode"], sec["kexp"])
            v = mxfp4.mx_decode(sec["vcode"], sec["vexp"])
        return (np.asarray(k, dtype=np.float32).reshape(shape), np.asarray(v, dtype=np.float32).reshape(shape))

    def sequence_tokens(self, block_row, length, kv_head):
        """Dequantized tokens 0..length-1 of one sequence and kv-head, read
        through its block-table row.  Returns (k_hat_rot, v_hat) as fp64
        [length, D]; keys stay in the rotated domain."""
        nblk = -(-int(length) // BLOCK)
        if nblk == 0:
            return np.zeros((0, self.d)), np.zeros((0, self.d))
        ids = np.asarray(block_row[:nblk], dtype=np.int64)
        recs = self.pool[ids, kv_head]
        if self.fmt in (FORMAT_TQ4, FORMAT_TQ4V2):
            sec = (layout.tq4_read_block if self.fmt == FORMAT_TQ4 else layout.tq4v2_read_block)(recs, self.d)
            k = tq4.key_dequant_rot(sec["kcode"], sec["kscale"], self.table)
            v = tq4.value_dequant(sec["vcode"], sec["vscale"], sec["vmin"])
        else:
            sec = layout.mxfp4_read_block(recs, self.d)
            k = mxfp4.mx_decode(sec["kcode"], sec["kexp"])
            v = mxfp4.mx_decode(sec["vcode"], sec["vexp"])
        k = np.asarray(k, dtype=np.float64).reshape(nblk * BLOCK, self.d)[:length]
        v = np.asarray(v, dtype=np.float64).reshape(nblk * BLOCK, self.d)[:length]
        return k, v
