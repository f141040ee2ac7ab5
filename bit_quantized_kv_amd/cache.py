"""Convenience wrapper: a cache whose pool and decode workspace are torch
tensors on the current device.  Marshalling only."""
import torch

from . import binding as B


class Cache:
    def __init__(self, fmt, head_dim, num_kv_heads, num_blocks, key_table=None, device="cuda"):
        self.fmt, self.head_dim, self.num_kv_heads, self.num_blocks = fmt, head_dim, num_kv_heads, num_blocks
        nbytes = B.tq_pool_bytes(fmt, head_dim, num_kv_heads, num_blocks)
        self.pool = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.handle = B.tq_create_cache(fmt, head_dim, num_kv_heads, num_blocks, key_table, self.pool)
        self.record_bytes = B.tq_record_bytes(fmt, head_dim, num_kv_heads, num_blocks)
        self._ws = None
        self._mt_ws = None
        self._cas_ws = None

    def quantize_append(self, k, v, slot_mapping, stream=None):
        assert k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16 and slot_mapping.dtype == torch.int32
        assert k.is_contiguous() and v.is_contiguous() and slot_mapping.is_contiguous()
        assert k.shape == v.shape and k.shape[1:] == (self.num_kv_heads, self.head_dim)
        assert slot_mapping.shape == (k.shape[0],)
        B.tq_quantize_append(self.handle, k, v, slot_mapping, stream)

    def workspace(self, batch, num_q_heads, max_context_len):
        need = B.tq_decode_workspace_bytes(self.handle, batch, num_q_heads, max_context_len)
        if need == 0:
            return None
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.pool.device)
        return self._ws

    def decode(self, q, block_table, context_lens, max_context_len, softmax_scale, out=None,
               out_dtype=torch.float32, stream=None):
        assert q.dtype == torch.bfloat16 and q.is_contiguous() and q.shape[2] == self.head_dim
        assert block_table.dtype == torch.int32 and block_table.is_contiguous()
        assert context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],)
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        ws = self.workspace(q.shape[0], q.shape[1], max_context_len)
        B.tq_decode_attention(self.handle, q, out, block_table, context_lens, max_context_len, softmax_scale, ws,
                              stream)
        return out

    def dequantize(self, block_ids, stream=None):
        """Test-only: the dequantized records of ``block_ids`` (device int32
        [n]) as (k_hat_rot, v_hat) float32 [n, Hkv, 16, D] device tensors."""
        n = int(block_ids.numel())
        k = torch.empty((n, self.num_kv_heads, 16, self.head_dim), dtype=torch.float32, device=self.pool.device)
        v = torch.empty_like(k)
        B.tq_debug_dequantize(self.handle, block_ids, k, v, stream)
        return k, v

    def key_table_f16(self):
        return B.tq_cache_info(self.handle)[2]

    def close(self):
        if self.handle is not None:
            B.tq_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def multitoken(self, q, q_start, max_query_len, block_table, context_lens, max_context_len, softmax_scale,
                   out=None, out_dtype=None, stream=None):
        """Causal attention of q [num_tokens, Hq, D] (sequence b's tokens are
        q[q_start[b]:q_start[b+1]], the last ones of its context)."""
        assert q.dtype == torch.bfloat16 and q.is_contiguous() and q.shape[2] == self.head_dim
        assert q_start.dtype == torch.int32 and context_lens.dtype == torch.int32
        n, hq, d = q.shape
        batch = int(q_start.numel()) - 1
        if out is None:
            out = torch.empty((n, hq, d), dtype=out_dtype or torch.float32, device=q.device)
        need = B.tq_multitoken_workspace_bytes(self.handle, batch, hq, n, max_query_len, max_context_len)
        ws = None
        if need:
            if self._mt_ws is None or self._mt_ws.numel() < need:
                self._mt_ws = torch.empty(need, dtype=torch.uint8, device=self.pool.device)
            ws = self._mt_ws
        B.tq_multitoken_attention(self.handle, q, out, q_start, max_query_len, block_table, context_lens,
                                  max_context_len, softmax_scale, ws, stream)
        return out

    def cascade_decode(self, q, block_table, context_lens, max_context_len, softmax_scale, groups, out=None,
                       out_dtype=torch.float32, stream=None):
        """Decode attention reading each group's shared blocks once
        (``groups``: a CascadeGroups)."""
        assert q.dtype == torch.bfloat16 and q.is_contiguous() and q.shape[2] == self.head_dim
        assert block_table.dtype == torch.int32 and context_lens.dtype == torch.int32
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        need = B.tq_cascade_workspace_bytes(self.handle, q.shape[0], q.shape[1], max_context_len, groups.num_groups,
                                            groups.max_group_size, groups.max_group_blocks, groups.max_depth)
        if self._cas_ws is None or self._cas_ws.numel() < need:
            self._cas_ws = torch.empty(need, dtype=torch.uint8, device=self.pool.device)
        B.tq_cascade_decode_attention(self.handle, q, out, block_table, context_lens, max_context_len, softmax_scale,
                                      groups, self._cas_ws, stream)
        return out


class CascadeGroups:
    """Shared-block groups for cascade decode, as device int32 tensors.
    ``groups``: list of (member sequences, lo, hi) block ranges whose members'
    block tables agree on blocks lo .. hi - 1; the groups of a sequence must
    cover its first blocks contiguously from 0.  A range longer than
    ``max_blocks`` is cut into chained groups of that many blocks (a group is
    one unit of parallel work), and a group of more than ``max_members``
    sequences (if given) into groups of at most that many over the same range:
    at most 32 rows (members times query heads per kv-head) per group take the
    library's direct kernel, which runs every row of a group on each wave.
    Marshalling only: depths, per-sequence block counts and the bounds follow
    from the list."""

    def __init__(self, batch, groups, max_blocks=48, max_members=None, device="cuda"):
        i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=device)
        cut = []
        for members, lo, hi in groups:
            members = list(members)
            step = max_members or max(1, len(members))
            for m0 in range(0, len(members), step):
                for s in range(lo, hi, max_blocks):
                    cut.append((members[m0:m0 + step], s, min(hi, s + max_blocks)))
        groups = cut
        pb = [0] * batch
        depth = [0] * batch
        starts, seqs, blocks, gdepth = [0], [], [], []
        for members, lo, hi in sorted(groups, key=lambda g: g[1]):
            d = depth[members[0]]
            for b in members:
                if pb[b] != lo or depth[b] != d:
                    raise ValueError("a sequence's groups must cover its blocks contiguously from 0")
                pb[b] = hi
                depth[b] = d + 1
            seqs += list(members)
            starts.append(len(seqs))
            blocks += [lo, hi]
            gdepth.append(d)
        self.num_groups = len(groups)
        self.max_group_size = max([len(g[0]) for g in groups] + [1])
        self.max_group_blocks = max([g[2] - g[1] for g in groups] + [0])
        self.max_depth = max(depth + [0]) if groups else 0
        self.seq_prefix_blocks = i32(pb)
        self.seq_depth = i32(depth)
        self.group_start = i32(starts)
        self.group_seqs = i32(seqs or [0])
        self.group_blocks = i32(blocks or [0, 0])
        self.group_depth = i32(gdepth or [0])


def calibrate_key_tables(k, init_table=None, max_iters=100, stream=None):
    """Fit one key table per layer on calibration keys ``k`` (device bf16
    [layers, rows, head_dim]).  Returns device tensors (tables int16 fp16
    bits [layers, 16], levels float64 [layers, 16], mse float64 [layers, 2],
    updates int32 [layers]).  Marshalling only: the fit runs in the library."""
    layers, rows, d = k.shape
    dev = k.device
    tables = torch.empty((layers, 16), dtype=torch.int16, device=dev)
    levels = torch.empty((layers, 16), dtype=torch.float64, device=dev)
    mse = torch.empty((layers, 2), dtype=torch.float64, device=dev)
    updates = torch.empty((layers,), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, B.tq_calibrate_workspace_bytes(layers, rows, d)), dtype=torch.uint8, device=dev)
    B.tq_calibrate_key_tables(k, init_table, max_iters, tables, levels, mse, updates, ws, stream)
    return tables, levels, mse, updates
