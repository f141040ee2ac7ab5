"""Pins for oracle.attention and oracle.paged: brute force, invariants, merge."""
import math

import numpy as np

from oracle import attention, lloyd_max, paged, tq4, wht
import workloads


def _brute(q, k, v, scale):
    """Pure-Python loops, fp64."""
    T = len(k)
    logits = [scale * sum(q[i] * k[t][i] for i in range(len(q))) for t in range(T)]
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    s = sum(e)
    return [sum(e[t] / s * v[t][j] for t in range(T)) for j in range(len(v[0]))]


def test_softmax_attention_vs_brute_force():
    rng = np.random.default_rng(20)
    q = rng.standard_normal(8)
    k = rng.standard_normal((13, 8))
    v = rng.standard_normal((13, 8))
    o, w = attention.softmax_attention(q, k, v, 0.7)
    assert np.allclose(o, _brute(q.tolist(), k.tolist(), v.tolist(), 0.7), rtol=1e-13, atol=1e-14)
    assert abs(w.sum() - 1) < 1e-12


def test_special_cases():
    rng = np.random.default_rng(21)
    v = rng.standard_normal((9, 4))
    o, _ = attention.softmax_attention(rng.standard_normal(4), rng.standard_normal((1, 4)), v[:1], 0.5)
    assert np.allclose(o, v[0], rtol=0, atol=0)                      # T = 1
    o, _ = attention.softmax_attention(np.zeros(4), rng.standard_normal((9, 4)), v, 0.5)
    assert np.allclose(o, v.mean(0), rtol=1e-14)                     # equal logits -> mean
    o, _ = attention.softmax_attention(np.zeros(4), np.zeros((0, 4)), np.zeros((0, 4)), 0.5)
    assert np.all(o == 0)                                            # T = 0


def test_merge_of_any_partition_equals_single_pass():
    rng = np.random.default_rng(22)
    logits = rng.standard_normal(500) * 4
    v = rng.standard_normal((500, 16))
    ref = attention.merge([attention.partial_state(logits, v)])
    w = np.exp(logits - logits.max())
    assert np.allclose(ref, w @ v / w.sum(), rtol=1e-13)
    for _ in range(20):
        cuts = np.sort(rng.choice(np.arange(1, 500), size=rng.integers(1, 30), replace=False))
        parts = np.split(np.arange(500), cuts)
        states = [attention.partial_state(logits[p], v[p]) for p in parts] + [attention.partial_state([], v[:0])]
        assert np.max(np.abs(attention.merge(states) - ref)) < 1e-12


def _filled_pool(cfg):
    w = workloads.make(cfg)
    c = w.cfg
    pool = paged.PagedPool(c.fmt, w.num_blocks, c.num_kv_heads, c.head_dim)
    for b, t0, t1 in w.write_plan(w.total_lens):
        k, v = w.sequence_kv(b)
        pool.append(workloads.bf16_bits_to_f32(k[t0:t1]), workloads.bf16_bits_to_f32(v[t0:t1]), w.slots(b, t0, t1))
    return w, pool


def test_decode_matches_brute_force_over_dequantized_rows():
    cfg = workloads.small_config(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, ctx_range=(5, 40), seed=23)
    w, pool = _filled_pool(cfg)
    q = workloads.bf16_bits_to_f32(w.query_bits())
    out = attention.decode(pool, q, w.block_table, w.context_lens_at(), cfg.scale)
    table = lloyd_max.default_key_table_f16()
    for b in range(2):
        T = int(w.context_lens_at()[b])
        k, v = w.sequence_kv(b)
        k = workloads.bf16_bits_to_f32(k)[:T]
        v = workloads.bf16_bits_to_f32(v)[:T]
        for h in range(4):
            kvh = h // 2
            s = tq4.key_scale(k[:, kvh])
            kc = tq4.key_codes(k[:, kvh], s, table)
            kr = tq4.key_dequant_rot(kc, s, table).astype(np.float64)
            vc, sc, mn = tq4.value_encode(v[:, kvh])
            vh = tq4.value_dequant(vc, sc, mn).astype(np.float64)
            # unrotate the dequantized keys and use the unrotated query: same logits
            k_unrot = wht.wht_f64(kr)
            ref = _brute(q[b, h].astype(np.float64).tolist(), k_unrot.tolist(), vh.tolist(), cfg.scale)
            assert np.allclose(out[b, h], ref, rtol=1e-10, atol=1e-12)


def test_gqa_g1_is_per_head_attention():
    cfg = workloads.small_config(batch=1, num_q_heads=2, num_kv_heads=2, head_dim=64, ctx_range=(30, 30), seed=24)
    w, pool = _filled_pool(cfg)
    q = workloads.bf16_bits_to_f32(w.query_bits())
    out = attention.decode(pool, q, w.block_table, w.context_lens_at(), cfg.scale)
    for h in range(2):
        k, v = pool.sequence_tokens(w.block_table[0], 30, h)
        o, _ = attention.softmax_attention(wht.wht_f64(q[0, h]), k, v, cfg.scale)
        assert np.allclose(out[0, h], o, rtol=1e-14)


def test_permuted_block_table_gives_identical_tokens():
    base = workloads.small_config(batch=2, head_dim=128, ctx_range=(100, 180), seed=25, identity_table=True)
    perm = workloads.small_config(batch=2, head_dim=128, ctx_range=(100, 180), seed=25, identity_table=False)
    w1, p1 = _filled_pool(base)
    w2, p2 = _filled_pool(perm)
    assert not np.array_equal(w1.block_table, w2.block_table)
    for b in range(2):
        T = int(w1.total_lens[b])
        for h in range(2):
            k1, v1 = p1.sequence_tokens(w1.block_table[b], T, h)
            k2, v2 = p2.sequence_tokens(w2.block_table[b], T, h)
            assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_shared_prefix_blocks_are_read_by_every_sharer():
    cfg = workloads.small_config(batch=3, head_dim=64, ctx_range=(70, 90), shared_seqs=2, shared_tokens=48, seed=26)
    w, pool = _filled_pool(cfg)
    assert np.array_equal(w.block_table[0, :3], w.block_table[1, :3])
    k0, _ = pool.sequence_tokens(w.block_table[0], 48, 0)
    k1, _ = pool.sequence_tokens(w.block_table[1], 48, 0)
    assert np.array_equal(k0, k1)


def test_skip_and_duplicate_slots():
    pool = paged.PagedPool(0, 2, 1, 64)
    rng = np.random.default_rng(27)
    k = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal((3, 1, 64)).astype(np.float32)))
    pool.append(k, k, np.array([-1, 5, 5]))
    assert np.all(pool.pool[1] == 0)
    ref = paged.PagedPool(0, 2, 1, 64)
    ref.append(k[2:], k[2:], np.array([5]))
    assert np.array_equal(pool.pool, ref.pool)


def test_context_zero_gives_zero_row():
    cfg = workloads.small_config(batch=1, num_q_heads=2, num_kv_heads=1, head_dim=64, ctx_range=(16, 16), seed=28)
    w, pool = _filled_pool(cfg)
    q = workloads.bf16_bits_to_f32(w.query_bits())
    out = attention.decode(pool, q, w.block_table, np.zeros(1, np.int32), cfg.scale)
    assert np.all(out == 0)


def _multi_token_case(seed, lens_m, d=64, hq=8, hkv=2):
    cfg = workloads.small_config(batch=len(lens_m), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                 ctx_range=(20, 90), seed=seed)
    w, pool = _filled_pool(cfg)
    m = np.array([min(x, int(t)) for x, t in zip(lens_m, w.total_lens)])
    q_start = np.concatenate([[0], np.cumsum(m)])
    rng = np.random.default_rng(seed)
    q = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(
        rng.standard_normal((int(q_start[-1]), hq, d)).astype(np.float32)))
    return cfg, w, pool, m, q_start, q


def test_multi_token_rows_equal_decode_over_each_causal_prefix():
    cfg, w, pool, m, q_start, q = _multi_token_case(29, [1, 5, 17])
    T = w.total_lens
    out = attention.multi_token(pool, q, q_start, w.block_table, T, cfg.scale)
    for b in range(cfg.batch):
        for i in range(int(m[b])):
            qi = int(q_start[b]) + i
            ctx = np.array([int(T[b]) - int(m[b]) + i + 1])
            ref = attention.decode(pool, q[qi][None], w.block_table[b:b + 1], ctx, cfg.scale)
            assert np.array_equal(out[qi], ref[0])


def test_multi_token_against_masked_softmax_matrix():
    from scipy.special import softmax
    cfg, w, pool, m, q_start, q = _multi_token_case(30, [9], hq=2, hkv=1)
    T, M = int(w.total_lens[0]), int(m[0])
    out = attention.multi_token(pool, q, q_start, w.block_table, w.total_lens, cfg.scale)
    k, v = pool.sequence_tokens(w.block_table[0], T, 0)
    for h in range(2):
        qr = wht.wht_f64(q[:, h].astype(np.float64))                  # [M, D]
        s = cfg.scale * qr @ k.T                                        # [M, T]
        pos = np.arange(T)[None, :]
        s = np.where(pos > (T - M + np.arange(M))[:, None], -np.inf, s)
        ref = softmax(s, axis=1) @ v
        assert np.allclose(out[:, h], ref, rtol=1e-12, atol=1e-13)


def test_multi_token_prefill_from_the_first_token():
    # M = T: the first query token sees only token 0, so its output is v_hat[0]
    cfg, w, pool, m, q_start, q = _multi_token_case(31, [10 ** 6, 3])
    T0 = int(w.total_lens[0])
    assert int(m[0]) == T0
    out = attention.multi_token(pool, q, q_start, w.block_table, w.total_lens, cfg.scale,
                                rows=[(0, h) for h in range(cfg.num_q_heads)])
    for h in range(cfg.num_q_heads):
        _, v = pool.sequence_tokens(w.block_table[0], T0, h // 4)
        assert np.array_equal(out[0, h], v[0])


def test_cascade_decode_equals_decode():
    cfg = workloads.small_config(batch=5, num_q_heads=8, num_kv_heads=2, head_dim=64, ctx_range=(70, 200),
                                 shared_seqs=3, shared_tokens=64, seed=32)
    w, pool = _filled_pool(cfg)
    assert np.array_equal(w.block_table[0, :4], w.block_table[2, :4])
    q = workloads.bf16_bits_to_f32(w.query_bits())
    ctx = w.context_lens_at()
    ref = attention.decode(pool, q, w.block_table, ctx, cfg.scale)
    # the true sharing (4 blocks), a shorter claimed prefix, nested groups and
    # a one-member group
    for groups in ([([0, 1, 2], 0, 4)], [([0, 1, 2], 0, 2), ([4], 0, 3)],
                   [([0, 1, 2], 0, 1), ([0, 2], 1, 3), ([2], 3, 4)]):
        out = attention.cascade_decode(pool, q, w.block_table, ctx, cfg.scale, groups)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
