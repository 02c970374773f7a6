"""GPU cache write (pa_reshape_and_cache) against the oracle, bit for bit.

[INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理" (jsqmd.com), §1.2 and §3.3
"""

import numpy as np
import pytest
import torch

import oracle.paged_attention as O
from paged_kv_cache_362_amd import layouts, ops

pytestmark = pytest.mark.gpu


def _bits(x: torch.Tensor) -> np.ndarray:
    x = x.detach().cpu().contiguous()
    return x.view(torch.int32 if x.element_size() == 4 else torch.int16).numpy()


def _write_and_compare(b: layouts.PagedBatch):
    t = layouts.to_device(b)
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_cache"], t["v_cache"],
                          t["slot_mapping"])
    torch.cuda.synchronize()
    kc, vc = O.ref_reshape_and_cache(b.new_key, b.new_value, b.k_cache, b.v_cache,
                                     b.slot_mapping)
    # compare bit patterns of the whole pools (NaN payloads included)
    view = np.int32 if b.dtype == "f32" else np.int16
    assert np.array_equal(_bits(t["k_cache"]), kc.view(view)), "K pool differs"
    assert np.array_equal(_bits(t["v_cache"]), vc.view(view)), "V pool differs"
    return t


def test_config1_fresh_block_write():
    """The 51st token of config 1 goes to offset 0 of the next free block."""
    b = layouts.make_config(1, poison=True)
    fresh = int(b.slot_mapping[0]) // b.block_size
    assert fresh not in b.block_tables[0].tolist()
    t = _write_and_compare(b)
    got = t["k_cache"][fresh, :, 0, :].cpu().numpy()
    assert np.array_equal(got, b.new_key[0])


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_config_write(cfg):
    _write_and_compare(layouts.make_config(cfg, poison=True))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bs", [8, 16, 32, 64])
def test_shapes(dtype, d, bs):
    lens = np.array([1, bs, bs + 1, 3 * bs - 1, 100], np.int32)
    b = layouts.make_paged_batch(num_q_heads=4, num_kv_heads=2, head_dim=d, dtype=dtype,
                                 block_size=bs, context_lens=lens, seed=d + bs, poison=True)
    _write_and_compare(b)


def test_negative_and_out_of_range_slots_write_nothing():
    b = layouts.scaled_config(2, max_seqs=4, max_len=300)
    b.slot_mapping = b.slot_mapping.copy()
    b.slot_mapping[1] = -1
    t = layouts.to_device(b)
    before_k = _bits(t["k_cache"]).copy()
    kc, _ = O.ref_reshape_and_cache(b.new_key, b.new_value, b.k_cache, b.v_cache, b.slot_mapping)
    # a slot past the pool is skipped by the kernel (and reported under PA_DEBUG)
    t["slot_mapping"][2] = b.num_blocks * b.block_size + 3
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_cache"], t["v_cache"],
                          t["slot_mapping"])
    torch.cuda.synchronize()
    after = _bits(t["k_cache"])
    expect = kc.view(np.int16).copy()
    s2 = int(b.slot_mapping[2])
    expect[s2 // b.block_size, :, s2 % b.block_size, :] = \
        before_k[s2 // b.block_size, :, s2 % b.block_size, :]
    assert np.array_equal(after, expect)


def test_many_tokens_one_launch():
    """Prefill-sized write: 4096 tokens scattered over a shuffled pool."""
    rng = np.random.default_rng(8)
    n, hkv, d, bs = 4096, 8, 128, 16
    nb = n // bs + 40
    perm = rng.permutation(nb)
    slots = (perm[np.arange(n) // bs] * bs + np.arange(n) % bs).astype(np.int32)
    key = layouts.draw(rng, (n, hkv, d), "bf16")
    val = layouts.draw(rng, (n, hkv, d), "bf16")
    kc = layouts.draw(rng, (nb, hkv, bs, d), "bf16")
    vc = layouts.draw(rng, (nb, hkv, bs, d), "bf16")
    b = layouts.PagedBatch(dtype="bf16", num_q_heads=hkv, num_kv_heads=hkv, head_dim=d,
                           block_size=bs, q=np.zeros((1, hkv, d), np.uint16), k_cache=kc,
                           v_cache=vc, block_tables=np.zeros((1, 1), np.int32),
                           context_lens=np.ones(1, np.int32), new_key=key, new_value=val,
                           slot_mapping=slots, scale=1.0, seed=8, poisoned=False,
                           unique_blocks=nb)
    _write_and_compare(b)
