"""Exact decode attention over the dequantized paged cache, and the split/merge
(log-sum-exp) algebra.

Test infrastructure only (see ``oracle/__init__``).

Decode attention (one query token per sequence) is the step whose memory
traffic the 4-bit cache shrinks ([UQ] "這篇論文在解什麼痛點": KV cache fills
HBM; "方法怎麼做，白話講": decode reads the compressed cache; [TQ-AMD]
section 1: the aim is smaller KV with throughput kept).  The pages state no
formula; the reading is standard softmax attention:

  o[b, h] = sum_{t < T_b} softmax_t( scale * <q~[b,h], k_hat[b, h // g, t]> ) v_hat[b, h // g, t]

* g = Hq / Hkv, query head h uses kv-head h // g (contiguous grouping);
* keys are compared in the rotated domain: q~ = H_D q in fp64 for TQ4/4 (the
  rotation is orthonormal, so this equals q . k for unrotated keys);
  for MX-FP4 q~ is the query's own e4m3 code value (the rotated query as the
  kernels store it);
* T_b = 0 gives a zero row; no other mask (the new token is already cached).

Several query tokens per sequence (``multi_token``: chunked prefill, or the
verification of proposed tokens) take the standard causal reading: the query
tokens are the last ones of the context, and each sees the keys up to its own
position.

All arithmetic is fp64.  Pinned by tests/test_oracle_attention.py: weights sum
to 1, brute-force loops on tiny inputs, T = 1, equal logits, merge of any
partition equals the single pass, GQA with g = 1 equals per-head MHA, block
table permutation invariance; multi_token against decode over each causal
prefix and against an explicitly masked softmax matrix; cascade_decode
against decode.
"""
import numpy as np

from . import fpformats as fp
from . import mxfp4, paged, wht


def softmax_attention(q_rot, k_rot, v, scale):
    """One query row against T cached rows, fp64.  Returns (o, weights)."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    k_rot = np.asarray(k_rot, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k_rot.shape[0] == 0:
        return np.zeros(v.shape[-1]), np.zeros(0)
    logits = scale * (k_rot @ q_rot)
    m = logits.max()
    w = np.exp(logits - m)
    w = w / w.sum()
    return w @ v, w


def decode(pool, q, block_table, context_lens, scale, rows=None):
    """Decode attention for every (b, h) (or only ``rows``, a list of (b, h)).

    ``pool`` is a ``paged.PagedPool``; ``q`` fp32 [B, Hq, D] holding bf16
    values.  Returns fp64 [B, Hq, D] (rows not requested are NaN)."""
    q = np.asarray(q, dtype=np.float32)
    bsz, hq, d = q.shape
    if hq % pool.hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = hq // pool.hkv
    out = np.full((bsz, hq, d), np.nan)
    want = rows if rows is not None else [(b, h) for b in range(bsz) for h in range(hq)]
    cache = {}
    for b, h in want:
        kvh = h // g
        key = (b, kvh)
        if key not in cache:
            cache[key] = pool.sequence_tokens(block_table[b], int(context_lens[b]), kvh)
        k_rot, v_hat = cache[key]
        out[b, h] = softmax_attention(rotated_query(pool, q[b, h]), k_rot, v_hat, scale)[0]
    return out


def multi_token(pool, q, q_start, block_table, context_lens, scale, rows=None):
    """Attention of several query tokens per sequence over the cache: chunked
    prefill of new tokens, or the verification of several proposed tokens.

    Sequence b's query tokens are q[q_start[b] : q_start[b+1]], the last
    M_b = q_start[b+1] - q_start[b] tokens of its context of T_b tokens
    (their keys and values are already in the cache).  Query token i of the
    sequence sits at position T_b - M_b + i and, causally, sees the keys at
    positions t < T_b - M_b + i + 1.  Each row is ``softmax_attention`` over
    that prefix; M_b = 1 is ``decode``.

    ``q`` fp32 [total_q, Hq, D] holding bf16 values; ``rows`` a list of
    (query token index into q, head) or None for all.  Returns fp64
    [total_q, Hq, D] (rows not requested are NaN)."""
    q = np.asarray(q, dtype=np.float32)
    total, hq, d = q.shape
    if hq % pool.hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    g = hq // pool.hkv
    q_start = np.asarray(q_start, dtype=np.int64)
    seq_of = np.zeros(total, dtype=np.int64)
    for b in range(len(q_start) - 1):
        seq_of[q_start[b]:q_start[b + 1]] = b
    out = np.full((total, hq, d), np.nan)
    want = rows if rows is not None else [(i, h) for i in range(total) for h in range(hq)]
    cache = {}
    for qi, h in want:
        b = int(seq_of[qi])
        tb = int(context_lens[b])
        mb = int(q_start[b + 1] - q_start[b])
        visible = tb - mb + (qi - int(q_start[b])) + 1
        if visible < 1 or visible > tb:
            raise ValueError("each query token must lie inside its sequence's context")
        kvh = h // g
        key = (b, kvh)
        if key not in cache:
            cache[key] = pool.sequence_tokens(block_table[b], tb, kvh)
        k_rot, v_hat = cache[key]
        out[qi, h] = softmax_attention(rotated_query(pool, q[qi, h]), k_rot[:visible], v_hat[:visible], scale)[0]
    return out


def cascade_decode(pool, q, block_table, context_lens, scale, groups, rows=None):
    """Decode attention computed the cascade way, for sequences that share
    leading blocks ([UQ] "它實際證明了什麼" and [TQ-AMD] spec table: agentic
    sessions with long shared prefixes).

    ``groups``: list of (member sequences, lo, hi): the members' tables agree
    on blocks lo .. hi - 1, and a sequence's groups cover its first blocks
    contiguously from 0.  For a row of member b, the partial state (max, sum,
    acc) over each of its groups' tokens (read through the group's first
    member's table, once for the group) and the state over its own remaining
    tokens are combined by ``merge``; other sequences are plain ``decode``
    rows.  By the merge identity the result equals ``decode``.  Returns fp64
    [B, Hq, D] (rows not requested are NaN)."""
    q = np.asarray(q, dtype=np.float32)
    bsz, hq, d = q.shape
    g = hq // pool.hkv
    of_seq = {}
    for members, lo, hi in groups:
        for b in members:
            of_seq.setdefault(int(b), []).append((int(lo), int(hi), int(members[0])))
    out = np.full((bsz, hq, d), np.nan)
    want = rows if rows is not None else [(b, h) for b in range(bsz) for h in range(hq)]
    for b, h in want:
        tb = int(context_lens[b])
        kvh = h // g
        k_rot, v_hat = pool.sequence_tokens(block_table[b], tb, kvh)
        qr = rotated_query(pool, q[b, h])
        states, own = [], 0
        for lo, hi, first in sorted(of_seq.get(b, [])):
            if lo != own:
                raise ValueError("a sequence's groups must cover its blocks contiguously from 0")
            k_sh, v_sh = pool.sequence_tokens(block_table[first], 16 * hi, kvh)
            states.append(partial_state(scale * (k_sh[16 * lo:] @ qr), v_sh[16 * lo:]))
            own = hi
        states.append(partial_state(scale * (k_rot[16 * own:] @ qr), v_hat[16 * own:]))
        out[b, h] = merge(states)
    return out


def rotated_query(pool, qrow):
    if pool.fmt in (paged.FORMAT_TQ4, paged.FORMAT_TQ4V2):
        return wht.wht_f64(qrow)
    return fp.e4m3_decode(mxfp4.query_fp8(qrow))


# --- split / merge -----------------------------------------------------------

def partial_state(logits, v):
    """(m, l, acc) of one chunk: m = max logit, l = sum exp(logit - m),
    acc = sum exp(logit - m) v.  An empty chunk is (-inf, 0, 0)."""
    logits = np.asarray(logits, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if logits.size == 0:
        return -np.inf, 0.0, np.zeros(v.shape[-1])
    m = logits.max()
    e = np.exp(logits - m)
    return m, e.sum(), e @ v


def merge(states):
    """Combine chunk states: M = max m_i, o = sum e^{m_i-M} acc_i / sum e^{m_i-M} l_i."""
    ms = np.array([s[0] for s in states], dtype=np.float64)
    if np.all(np.isneginf(ms)):
        return np.zeros(len(states[0][2]))
    big = ms.max()
    wts = np.where(np.isneginf(ms), 0.0, np.exp(ms - big))
    num = sum(w * s[2] for w, s in zip(wts, states))
    den = sum(w * s[1] for w, s in zip(wts, states))
    return num / den
