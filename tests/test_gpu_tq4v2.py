"""GPU parity of TQ4/2 (4-bit keys, 2-bit values) against the CPU oracle,
through the C ABI: packed records byte for byte, decode attention within 2e-3
(max over rows of ||o - o_ref||_inf / ||o_ref||_inf) of the oracle's exact
attention over the same dequantized cache."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import workloads
from gpu_common import Case, check_case, say, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu

V2 = 2


@pytest.fixture(autouse=True)
def _split_env():
    saved = os.environ.pop("TQ_SPLIT_BLOCKS", None)
    yield
    os.environ.pop("TQ_SPLIT_BLOCKS", None)
    if saved is not None:
        os.environ["TQ_SPLIT_BLOCKS"] = saved


@pytest.mark.parametrize("d,g,hkv,seed,split", [
    (128, 4, 2, 401, None), (128, 8, 1, 402, 4), (128, 1, 3, 403, None), (64, 2, 2, 404, 8), (64, 4, 1, 405, None),
])
def test_small_ragged(d, g, hkv, seed, split):
    if split:
        os.environ["TQ_SPLIT_BLOCKS"] = str(split)
    cfg = workloads.small_config(batch=5, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, ctx_range=(1, 700),
                                 seed=seed, fmt=V2)
    say(f"case: TQ4/2 small ragged d={d} g={g} hkv={hkv} seed={seed} split={split}")
    check_case(Case(cfg))


def test_unaligned_skipped_and_single_token_slots():
    cfg = workloads.small_config(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=128, ctx_range=(160, 160),
                                 seed=406, fmt=V2)
    w = workloads.make(cfg)
    from bit_quantized_kv_amd import Cache
    from oracle import paged
    k, v = w.sequence_kv(0)
    rng = np.random.default_rng(6)
    slots = rng.permutation(w.num_blocks * 16)[:160].astype(np.int32)
    slots[rng.choice(160, 20, replace=False)] = -1
    cache = Cache(V2, 128, 2, w.num_blocks)
    say("case: TQ4/2 permuted slots with skips, then one-token appends")
    cache.quantize_append(to_dev_bf16(k[:100]), to_dev_bf16(v[:100]), to_dev_i32(slots[:100]))
    for i in range(100, 160):
        cache.quantize_append(to_dev_bf16(k[i:i + 1]), to_dev_bf16(v[i:i + 1]), to_dev_i32(slots[i:i + 1]))
    torch.cuda.synchronize()
    gpu = cache.pool.cpu().numpy().reshape(w.num_blocks, 2, -1)
    op = paged.PagedPool(V2, w.num_blocks, 2, 128)
    op.append(workloads.bf16_bits_to_f32(k), workloads.bf16_bits_to_f32(v), slots)
    assert np.array_equal(gpu, op.pool)


def test_full_llama8b_shape():
    cfg = dataclasses.replace(workloads.CONFIGS["llama8b"], name="llama8b-tq4v2", fmt=V2)
    say("case: TQ4/2 on the llama8b layer shape (B=1, 32/8, D=128, T=32768), all rows")
    check_case(Case(cfg))
