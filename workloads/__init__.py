"""Seeded synthetic inputs for the 4-bit KV-cache path.

This module is the only one that both the CPU oracle (``oracle/``) and the GPU
path's tests and benchmark import.  It draws random numbers and builds block
tables; it holds none of the codec or attention arithmetic.

The pages measure on serving workloads that are not available here (a vLLM
multi-turn benchmark over ShareGPT conversations, 32 concurrent sessions:
[UQ] "它實際證明了什麼"; 100 agentic conversations at 32 concurrency with
~25K-token prefixes: [TQ-AMD] spec table).  These generators stand in for them
with the same shapes: long shared prefixes, 32 concurrent sequences, private
tails.  No dataset item is used or reproduced.

Distributions (all drawn in fp32 with numpy's PCG64, then rounded to bf16 with
round-to-nearest-even):
* K = N(0,1) + per-(kv-head, channel) bias N(0, bias_std^2), then a few outlier
  channels per kv-head multiplied by ``outlier_mult``;
* V, q = N(0,1).

Streams: ``SeedSequence(seed).spawn(batch + 2)``: child 0 = global draws in the
order outlier channels -> biases -> context lengths -> queries -> block
permutation; child 1 = the shared prefix; child 2 + b = sequence b.
"""
from dataclasses import dataclass, field

import numpy as np

BLOCK = 16


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int = 0                    # fixed context length (0: use ctx_range)
    ctx_range: tuple = ()               # inclusive uniform range of context lengths
    shared_seqs: int = 0                # sequences 0..shared_seqs-1 share a prefix
    shared_tokens: int = 0              # length of the shared prefix
    outliers: int = 0                   # outlier channels per kv-head in K
    outlier_mult: float = 20.0
    bias_std: float = 0.0               # per-channel K bias std
    decode_steps: int = 1               # decode steps (each after its append)
    appended: int = 0                   # tokens appended per sequence during the steps
    fmt: int = 0                        # 0 = TQ4/4, 1 = MX-FP4
    identity_table: bool = False
    seed: int = 0
    softmax_scale: float = field(default=0.0)
    # magnitude multipliers of the drawn K, V and q (1: the distributions
    # above; other values give the range edge cases of the parity tests)
    k_scale: float = 1.0
    v_scale: float = 1.0
    q_scale: float = 1.0

    @property
    def scale(self):
        return self.softmax_scale if self.softmax_scale else 1.0 / np.sqrt(self.head_dim)


CONFIGS = {
    "tiny": Config("tiny", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, context=256,
                   outliers=2, identity_table=True, seed=1001, softmax_scale=1.0 / 8.0),
    "llama8b": Config("llama8b", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, context=32768,
                      outliers=4, bias_std=0.5, seed=1002),
    "agentic": Config("agentic", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
                      ctx_range=(4096, 25600), shared_seqs=16, shared_tokens=24576,
                      outliers=4, bias_std=0.5, seed=1003),
    "longprefix": Config("longprefix", batch=8, num_q_heads=64, num_kv_heads=8, head_dim=128, context=25600,
                         outliers=4, bias_std=0.5, decode_steps=64, appended=64, seed=1004),
    "fp4": Config("fp4", batch=128, num_q_heads=64, num_kv_heads=8, head_dim=128, context=16384,
                  outliers=4, fmt=1, seed=1005),
}


# Multi-token attention workloads (chunked prefill, verification).  The query
# tokens are the last ``query_tokens`` of each sequence's context; their keys
# and values are part of the sequence's cached tokens.
MT_CONFIGS = {
    # verification of 8 proposed tokens per sequence on the agentic shape
    "verify": Config("verify", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     ctx_range=(4096, 25600), shared_seqs=16, shared_tokens=24576,
                     outliers=4, bias_std=0.5, seed=1007),
    # a 512-token prefill chunk per sequence on top of a 25088-token cached prefix
    "prefill": Config("prefill", batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, context=25600,
                      outliers=4, bias_std=0.5, seed=1008),
    # the same two steps over an MX-FP4 cache
    "verify_fp4": Config("verify_fp4", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         ctx_range=(4096, 25600), shared_seqs=16, shared_tokens=24576,
                         outliers=4, fmt=1, seed=1009),
    "prefill_fp4": Config("prefill_fp4", batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, context=25600,
                          outliers=4, fmt=1, seed=1010),
}
MT_QUERY_TOKENS = {"verify": 8, "prefill": 512, "verify_fp4": 8, "prefill_fp4": 512}


def f32_to_bf16_bits(x):
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Workload:
    """All inputs of one configuration, generated lazily per sequence."""

    def __init__(self, cfg: Config, scale_ctx=None):
        self.cfg = cfg
        c = cfg
        kids = np.random.SeedSequence(c.seed).spawn(c.batch + 2)
        self._kids = kids
        g = np.random.Generator(np.random.PCG64(kids[0]))
        d, hkv = c.head_dim, c.num_kv_heads
        # 1. outlier channels per kv-head
        self.outlier_idx = np.stack([np.sort(g.choice(d, size=c.outliers, replace=False))
                                     for _ in range(hkv)]) if c.outliers else np.zeros((hkv, 0), np.int64)
        # 2. per-channel biases
        self.bias = (g.normal(0.0, c.bias_std, size=(hkv, d)).astype(np.float32)
                     if c.bias_std > 0 else np.zeros((hkv, d), np.float32))
        # 3. context lengths (final lengths, after any appended tokens)
        if c.ctx_range:
            lo, hi = c.ctx_range
            self.prompt_lens = g.integers(lo, hi + 1, size=c.batch).astype(np.int64)
        else:
            self.prompt_lens = np.full(c.batch, c.context, dtype=np.int64)
        self.total_lens = self.prompt_lens + c.appended
        # 4. queries, one set per decode step
        qf = g.standard_normal(size=(c.decode_steps, c.batch, c.num_q_heads, d), dtype=np.float32)
        if c.q_scale != 1.0:
            qf *= np.float32(c.q_scale)
        self.q_bits = f32_to_bf16_bits(qf)
        # 5. block table and pool size
        self._build_table(g)

    # -- block table ------------------------------------------------------------
    def _build_table(self, g):
        c = self.cfg
        nblk = -(-self.total_lens // BLOCK)
        self.max_blocks = int(nblk.max())
        shared_blocks = -(-c.shared_tokens // BLOCK) if c.shared_seqs else 0
        uses_shared = np.zeros(c.batch, dtype=np.int64)
        if c.shared_seqs:
            uses_shared[: c.shared_seqs] = np.minimum(nblk[: c.shared_seqs],
                                                      -(-np.minimum(self.total_lens[: c.shared_seqs], c.shared_tokens) // BLOCK))
        private = nblk - uses_shared
        self.num_blocks = int(shared_blocks + private.sum())
        ids = np.arange(self.num_blocks) if c.identity_table else g.permutation(self.num_blocks)
        table = np.zeros((c.batch, self.max_blocks), dtype=np.int32)
        shared_ids = ids[:shared_blocks]
        nxt = shared_blocks
        for b in range(c.batch):
            u = int(uses_shared[b])
            table[b, :u] = shared_ids[:u]
            n = int(private[b])
            table[b, u:u + n] = ids[nxt:nxt + n]
            nxt += n
        self.block_table = table
        self.shared_block_count = shared_blocks
        self.uses_shared = uses_shared

    # -- token data ---------------------------------------------------------------
    def _draw_kv(self, gen, n):
        c = self.cfg
        k = gen.standard_normal(size=(n, c.num_kv_heads, c.head_dim), dtype=np.float32)
        v = gen.standard_normal(size=(n, c.num_kv_heads, c.head_dim), dtype=np.float32)
        k += self.bias[None]
        for h in range(c.num_kv_heads):
            k[:, h, self.outlier_idx[h]] *= np.float32(c.outlier_mult)
        if c.k_scale != 1.0:
            k *= np.float32(c.k_scale)
        if c.v_scale != 1.0:
            v *= np.float32(c.v_scale)
        return f32_to_bf16_bits(k), f32_to_bf16_bits(v)

    def shared_prefix(self):
        """bf16 bits (K, V) [shared_tokens, Hkv, D] of the shared prefix."""
        c = self.cfg
        gen = np.random.Generator(np.random.PCG64(self._kids[1]))
        return self._draw_kv(gen, c.shared_tokens)

    def sequence_kv(self, b):
        """bf16 bits (K, V) [total_len_b, Hkv, D] of sequence b, shared prefix
        included for the sharing sequences."""
        c = self.cfg
        total = int(self.total_lens[b])
        ns = int(min(total, c.shared_tokens)) if b < c.shared_seqs else 0
        gen = np.random.Generator(np.random.PCG64(self._kids[2 + b]))
        kp, vp = self._draw_kv(gen, total - ns)
        if ns == 0:
            return kp, vp
        ks, vs = self.shared_prefix()
        return np.concatenate([ks[:ns], kp]), np.concatenate([vs[:ns], vp])

    def private_start(self, b):
        """First token of sequence b that lives in a private block."""
        return int(self.uses_shared[b]) * BLOCK if b < self.cfg.shared_seqs else 0

    def prefix_writer(self):
        """The sharing sequence with the most shared blocks: it writes the
        whole shared prefix (or -1 when nothing is shared)."""
        if not self.cfg.shared_seqs:
            return -1
        return int(np.argmax(self.uses_shared[: self.cfg.shared_seqs]))

    def write_plan(self, lens=None):
        """(b, t0, t1) ranges that write every token any sequence reads exactly
        once: the prefix writer writes from token 0, every other sequence only
        its private tokens.  ``lens`` defaults to the prompt lengths."""
        lens = self.prompt_lens if lens is None else np.asarray(lens)
        wr = self.prefix_writer()
        plan = []
        for b in range(self.cfg.batch):
            t0 = 0 if b == wr else self.private_start(b)
            t1 = int(lens[b])
            if t1 > t0:
                plan.append((b, t0, t1))
        return plan

    def shared_block_groups(self, ctx=None):
        """The nested groups of shared blocks: list of (members, lo, hi).
        Sharer b holds P_b = floor(min(T_b, shared_tokens) / 16) full shared
        blocks (a partly used last shared block stays its own); with the
        distinct P values p_1 < p_2 < ..., group i covers blocks p_{i-1} ..
        p_i - 1 for the sharers with P_b >= p_i."""
        c = self.cfg
        ctx = self.total_lens if ctx is None else np.asarray(ctx)
        pb = {b: int(min(int(ctx[b]), c.shared_tokens)) // BLOCK for b in range(c.shared_seqs)}
        levels = sorted(set(v for v in pb.values() if v > 0))
        groups, lo = [], 0
        for hi in levels:
            members = [b for b in range(c.shared_seqs) if pb[b] >= hi]
            groups.append((members, lo, hi))
            lo = hi
        return groups

    def slots(self, b, t0, t1):
        """Slot of each token t in [t0, t1) of sequence b."""
        t = np.arange(t0, t1)
        return (self.block_table[b, t // BLOCK].astype(np.int64) * BLOCK + t % BLOCK).astype(np.int32)

    def query_bits(self, step=0):
        return self.q_bits[step]

    def multi_queries(self, m):
        """Query tokens of a multi-token attention step: ``m`` (an int or one
        count per sequence, each clipped to the sequence's length) query tokens
        per sequence, N(0,1) in bf16.  Returns (q bits [sum m, Hq, D],
        q_start [batch + 1]).  Drawn from a stream of their own, so the other
        draws are unchanged."""
        c = self.cfg
        m = np.broadcast_to(np.asarray(m, dtype=np.int64), (c.batch,))
        m = np.minimum(m, self.total_lens)
        q_start = np.concatenate([[0], np.cumsum(m)]).astype(np.int32)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([c.seed, 0x6D74])))
        qf = g.standard_normal(size=(int(q_start[-1]), c.num_q_heads, c.head_dim), dtype=np.float32)
        return f32_to_bf16_bits(qf), q_start

    def context_lens_at(self, step=0):
        """Context lengths seen by decode step ``step`` (its token appended)."""
        c = self.cfg
        if c.appended:
            return (self.prompt_lens + step + 1).astype(np.int32)
        return self.total_lens.astype(np.int32)


def make(name_or_cfg):
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    return Workload(cfg)


def calibration_keys(layers=32, tokens=20, num_kv_heads=8, head_dim=128, seed=1006):
    """Calibration keys of a stack of layers: bf16 bits [layers, tokens *
    num_kv_heads, head_dim] (rows token-major, then kv-head).

    About 20 captured vectors per layer stand in for one forward pass's keys
    ([UQ] "方法怎麼做，白話講").  Layers differ in shape so that their key
    MSEs differ: per layer, Student-t entries with df ~ U[3, 30], a per-(head,
    channel) bias N(0, 0.5^2), and 1-4 outlier channels per kv-head scaled by
    ~U[1, 60] (a strong outlier makes the rotated row nearly two-valued)."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((layers, tokens * num_kv_heads, head_dim), dtype=np.uint16)
    for layer in range(layers):
        df = g.uniform(3.0, 30.0)
        mult = np.float32(g.uniform(1.0, 60.0))
        nout = int(g.integers(1, 5))
        k = g.standard_t(df, size=(tokens, num_kv_heads, head_dim)).astype(np.float32)
        k += g.normal(0.0, 0.5, size=(num_kv_heads, head_dim)).astype(np.float32)[None]
        for h in range(num_kv_heads):
            k[:, h, g.choice(head_dim, size=nout, replace=False)] *= mult
        out[layer] = f32_to_bf16_bits(k.reshape(tokens * num_kv_heads, head_dim))
    return out


def small_config(name="small", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, ctx_range=(1, 200),
                 fmt=0, seed=7, shared_seqs=0, shared_tokens=0, outliers=2, bias_std=0.5, identity_table=False,
                 k_scale=1.0, v_scale=1.0, q_scale=1.0):
    """A small ragged configuration for parity tests (several tiles, a ragged tail)."""
    return Config(name, batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                  ctx_range=ctx_range, shared_seqs=shared_seqs, shared_tokens=shared_tokens, outliers=outliers,
                  bias_std=bias_std, fmt=fmt, seed=seed, identity_table=identity_table, k_scale=k_scale,
                  v_scale=v_scale, q_scale=q_scale)
