"""GPU parity of pa_decode (and the cache write feeding it) against the oracle.

Runs the HIP library through its C ABI (via the ctypes binding) on an MI355X.
Tolerances are those of tests/parity.py.

[INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理" (jsqmd.com)
[KVP]   "PagedAttention：KV Cache 的分页革命" (openeuler.csdn.net)
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.paged_attention as O
from paged_kv_cache_362_amd import layouts, ops
from parity import assert_decode_close, gpu_step, oracle_step

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def _report(name, rep):
    print(f"[parity] {name}: {rep}", flush=True)


# ---------------------------------------------------------------------------
# the five workloads, scaled down (every output compared) and at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("partition", [0, 64])
def test_scaled_config_parity(cfg, partition):
    b = layouts.scaled_config(cfg, poison=True, max_seqs=4, max_len=700)
    _, _, o64 = oracle_step(b)
    _, out = gpu_step(b, partition=partition)
    rep = assert_decode_close(layouts.from_device(out, b.dtype), o64, b.dtype, b.name)
    _report(f"{b.name} P={partition}", rep)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_config_parity(cfg):
    """Full-size workload, every sequence, both entry points:
    pa_reshape_and_cache followed by pa_decode (balanced form), and the fused
    pa_decode_step that the benchmark times, each on its own copy of the
    poisoned pools, against the oracle run over the whole batch. The two
    outputs are bit-identical, the pools equal the oracle's write bit for bit,
    and a rerun of the decode reproduces its output bit for bit. (The tiny
    workload's token goes into a fresh block outside its context: the fused
    step writes that slot and reads nothing from it.)"""
    b = layouts.make_config(cfg, poison=True)
    kc, vc, o64 = oracle_step(b)
    t, out = gpu_step(b)
    rep = assert_decode_close(layouts.from_device(out, b.dtype), o64, b.dtype,
                              f"{b.name} write + decode")
    _report(f"{b.name} write + decode, all {b.num_seqs} sequences", rep)
    out2 = ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                      t["context_lens"], b.scale, b.max_context_len)
    assert torch.equal(_bits(out), _bits(out2))
    del t
    # the fused step too; the tiny workload writes its token into a fresh block
    # outside its context, a slot the launch writes and does not read
    t_step = layouts.to_device(b)
    out_step = ops.decode_step(t_step["q"], t_step["new_key"], t_step["new_value"],
                               t_step["k_cache"], t_step["v_cache"], t_step["slot_mapping"],
                               t_step["block_tables"], t_step["context_lens"], b.scale,
                               b.max_context_len)
    torch.cuda.synchronize()
    rep = assert_decode_close(layouts.from_device(out_step, b.dtype), o64, b.dtype,
                              f"{b.name} decode_step")
    _report(f"{b.name} decode_step, all {b.num_seqs} sequences", rep)
    for name, pool, want in (("k", t_step["k_cache"], kc), ("v", t_step["v_cache"], vc)):
        got = layouts.from_device(pool, b.dtype)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), f"{name} pool"
    assert torch.equal(_bits(out), _bits(out_step))


def _bits(x):
    return x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16)


# ---------------------------------------------------------------------------
# the pages' worked examples
# ---------------------------------------------------------------------------

def _fixed_table_batch(table, n, dtype="f32", hq=4, hkv=4, d=64, bs=16, seed=5):
    """One sequence whose table is given; pool 16 blocks, others poisoned."""
    rng = np.random.default_rng(seed)
    num_blocks = 16
    q = layouts.draw(rng, (1, hq, d), dtype)
    kc = layouts.draw(rng, (num_blocks, hkv, bs, d), dtype)
    vc = layouts.draw(rng, (num_blocks, hkv, bs, d), dtype)
    live = np.zeros((num_blocks, bs), bool)
    for pos in range(n):
        live[table[pos // bs], pos % bs] = True
    nv = layouts.nan_value(dtype)
    blk, off = np.nonzero(~live)
    kc[blk, :, off, :] = nv
    vc[blk, :, off, :] = nv
    width = len(table) + 2
    bt = np.full((1, width), [b for b in range(num_blocks) if b not in table][0], np.int32)
    bt[0, :len(table)] = table
    return layouts.PagedBatch(
        dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, q=q,
        k_cache=kc, v_cache=vc, block_tables=bt, context_lens=np.array([n], np.int32),
        new_key=np.zeros((0, hkv, d), kc.dtype), new_value=np.zeros((0, hkv, d), kc.dtype),
        slot_mapping=np.zeros((0,), np.int32), scale=float(np.float32(1 / math.sqrt(d))),
        seed=seed, poisoned=True, unique_blocks=len(table), name=f"table {table} n={n}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_worked_example_block_table(dtype):
    g = json.load(open(os.path.join(GOLDEN, "worked_example_block_table.json")))
    b = _fixed_table_batch(g["table"], g["context_len"], dtype)
    o64 = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale, dtype)
    _, out = gpu_step(b, write=False)
    _report(b.name, assert_decode_close(layouts.from_device(out, dtype), o64, dtype, b.name))


def test_page_table_example():
    g = json.load(open(os.path.join(GOLDEN, "page_table_example.json")))
    b = _fixed_table_batch(g["table"], g["context_len"], "f16")
    o64 = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale, "f16")
    _, out = gpu_step(b, write=False)
    assert_decode_close(layouts.from_device(out, "f16"), o64, "f16", b.name)


def test_51st_token_written_then_attended():
    """Position 50 goes to block 12 offset 2 (slot 194); decode at n = 51."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example_block_table.json")))
    b = _fixed_table_batch(g["table"], 51, "f32")
    rng = np.random.default_rng(9)
    b.new_key = layouts.draw(rng, (1, 4, 64), "f32")
    b.new_value = layouts.draw(rng, (1, 4, 64), "f32")
    b.slot_mapping = np.array([O.slot_of(g["table"], 50, 16)], np.int32)
    assert b.slot_mapping[0] == g["position_50"]["slot"]
    b.k_cache[12, :, 2, :] = np.nan  # the write must land before the read
    b.v_cache[12, :, 2, :] = np.nan
    _, _, o64 = oracle_step(b)
    t, out = gpu_step(b)
    assert_decode_close(layouts.from_device(out, "f32"), o64, "f32", "51st token")


# ---------------------------------------------------------------------------
# shapes, lengths and partitions
# ---------------------------------------------------------------------------

SHAPES = [
    # dtype, Hq, Hkv, D, B
    ("f16", 8, 8, 128, 16), ("bf16", 8, 2, 128, 16), ("f32", 4, 4, 64, 16),
    ("f16", 8, 1, 64, 8), ("bf16", 16, 2, 64, 32), ("f16", 4, 2, 256, 64),
    ("f32", 8, 4, 128, 32), ("bf16", 2, 2, 256, 8), ("f32", 8, 1, 128, 16),
    ("f16", 32, 4, 128, 32), ("bf16", 8, 2, 128, 8), ("f16", 4, 2, 128, 8),
]
EDGE_LENS = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 255, 256, 257, 511, 513, 1000]


@pytest.mark.parametrize("dtype,hq,hkv,d,bs", SHAPES)
def test_shapes_and_ragged_lengths(dtype, hq, hkv, d, bs):
    lens = np.array(EDGE_LENS, np.int32)
    b = layouts.make_paged_batch(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                                 block_size=bs, context_lens=lens, seed=21, poison=True,
                                 extra_table_cols=2, name=f"{dtype} {hq}/{hkv} D{d} B{bs}")
    _, _, o64 = oracle_step(b)
    for partition in (0, 16, 48, 512):
        _, out = gpu_step(b, partition=partition)
        rep = assert_decode_close(layouts.from_device(out, dtype), o64, dtype,
                                  f"{b.name} P={partition}")
    _report(b.name, rep)


def test_long_context_max_partition():
    """A 65536-token sequence (longest tested), default and largest partition
    (64 blocks of 16 tokens)."""
    lens = np.array([65536, 3], np.int32)
    b = layouts.make_paged_batch(num_q_heads=8, num_kv_heads=8, head_dim=128, dtype="f16",
                                 block_size=16, context_lens=lens, seed=22, poison=False)
    _, _, o64 = oracle_step(b)
    for partition in (0, 1024):
        _, out = gpu_step(b, partition=partition)
        assert_decode_close(layouts.from_device(out, "f16"), o64, "f16", f"64K P={partition}")


# ---------------------------------------------------------------------------
# invariants and closed forms on the GPU
# ---------------------------------------------------------------------------

def test_block_permutation_is_bit_identical():
    b = layouts.scaled_config(2, max_seqs=4, max_len=700)
    _, out1 = gpu_step(b)
    perm = np.random.default_rng(3).permutation(b.num_blocks)
    kc = np.empty_like(b.k_cache)
    vc = np.empty_like(b.v_cache)
    kc[perm] = b.k_cache
    vc[perm] = b.v_cache
    b2 = layouts.PagedBatch(**{**b.__dict__, "k_cache": kc, "v_cache": vc,
                               "block_tables": perm[b.block_tables].astype(np.int32),
                               "slot_mapping": (perm[b.slot_mapping // b.block_size] * b.block_size
                                                + b.slot_mapping % b.block_size).astype(np.int32)})
    _, out2 = gpu_step(b2)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_poisoned_pads_do_not_change_output():
    clean = layouts.scaled_config(3, max_seqs=4, max_len=700, poison=False)
    dirty = layouts.scaled_config(3, max_seqs=4, max_len=700, poison=True)
    _, o1 = gpu_step(clean)
    _, o2 = gpu_step(dirty)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_constant_values_give_exactly_one():
    b = layouts.scaled_config(2, max_seqs=4, max_len=700)
    b.k_cache = b.k_cache.copy()
    b.v_cache = np.ones_like(b.v_cache)
    b.new_value = np.ones_like(b.new_value)
    for partition in (0, 64):
        _, out = gpu_step(b, partition=partition)
        assert torch.all(out == 1.0)


def test_single_token_returns_its_value_exactly():
    b = layouts.make_paged_batch(num_q_heads=8, num_kv_heads=4, head_dim=128, dtype="bf16",
                                 block_size=16, context_lens=np.array([1, 1, 1]), seed=4)
    _, out = gpu_step(b, write=False)
    v = layouts.to_device(b)["v_cache"]
    for s in range(3):
        blk = int(b.block_tables[s, 0])
        for h in range(8):
            assert torch.equal(out[s, h], v[blk, h // 2, 0])


def _score_pattern(pattern, n, d, dtype):
    """Per-position key magnitude t_i: with q rows of constant entries c and key rows
    of constant entries t_i, the score of position i is c * t_i * sqrt(d).

    Scores rise by about 3 (16-bit data) or 1.5 (f32 data) log2 units every 16
    tokens. f32 ramps are centred on zero and its spikes are lower: an f32 score
    near 130 in log2 units is itself resolved only to about 1.5e-5 (its spacing),
    which no f32 kernel could keep within the 1e-5 output bound."""
    i = np.arange(n, dtype=np.float64)
    f32 = dtype == "f32"
    step = (0.065 if f32 else 0.13) / math.sqrt(d)
    mid = (n - 1) / 2 if f32 else 0.0
    if pattern == "rising":
        return step * (i - mid)
    if pattern == "falling":
        return step * (n - 1 - i - mid)
    t = np.zeros(n)  # "spikes": flat, then a jump in the middle and a larger one near the end
    t[n // 2] = (12.0 if f32 else 40.0) / math.sqrt(d)
    t[max(n - 3, 0)] = (20.0 if f32 else 70.0) / math.sqrt(d)
    return t


@pytest.mark.parametrize("pattern", ["rising", "falling", "spikes"])
@pytest.mark.parametrize("dtype,hq,hkv,d", [("f16", 8, 2, 128), ("bf16", 8, 2, 128),
                                            ("f32", 4, 4, 64), ("f16", 4, 4, 64)])
def test_scores_that_move_the_maximum(pattern, dtype, hq, hkv, d):
    """Steadily rising scores make the kernel raise its reference maximum and
    rescale its sums many times (every few 16-token rounds), in full and in masked
    rounds; falling scores and isolated spikes cover the other orders. Each query
    head of a group has its own slope (c = 1, 1.25, 1.5, 1.75)."""
    lens = np.array([700, 333, 64, 17])
    b = layouts.make_paged_batch(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                                 block_size=16, context_lens=lens, seed=21)
    g = hq // hkv
    c = 1.0 + 0.25 * (np.arange(hq) % g)
    b.q = layouts.to_storage(np.broadcast_to(c[None, :, None], b.q.shape).astype(np.float32),
                             dtype)
    k = O.to_f64(b.k_cache, dtype).copy()
    for s, n in enumerate(lens):
        t = _score_pattern(pattern, int(n), d, dtype)
        for pos in range(int(n)):
            blk = b.block_tables[s, pos // 16]
            k[blk, :, pos % 16, :] = t[pos]
    b.k_cache = layouts.to_storage(k.astype(np.float32), dtype)
    o64 = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale,
                       dtype)
    dev = layouts.to_device(b, "cuda")
    for partition in (0, 64):
        _, out = gpu_step(b, partition=partition, dev=dev, write=False)
        rep = assert_decode_close(layouts.from_device(out, dtype), o64, dtype,
                                  f"{pattern} {dtype} G{g} D{d} P={partition}")
        _report(f"{pattern} {dtype} G{g} D{d} P={partition}", rep)


def test_gqa_matches_repeated_mha():
    """GQA with G=4 and MHA on the repeated KV heads agree with the same oracle values."""
    b = layouts.scaled_config(3, max_seqs=3, max_len=500)
    _, _, o64 = oracle_step(b)
    _, o_gqa = gpu_step(b)
    g = b.num_q_heads // b.num_kv_heads
    mha = layouts.PagedBatch(**{**b.__dict__, "num_kv_heads": b.num_q_heads,
                                "k_cache": np.repeat(b.k_cache, g, axis=1),
                                "v_cache": np.repeat(b.v_cache, g, axis=1),
                                "new_key": np.repeat(b.new_key, g, axis=1),
                                "new_value": np.repeat(b.new_value, g, axis=1)})
    _, o_mha = gpu_step(mha)
    assert_decode_close(layouts.from_device(o_gqa, "bf16"), o64, "bf16", "gqa")
    assert_decode_close(layouts.from_device(o_mha, "bf16"), o64, "bf16", "mha")


def test_split_matches_unsplit():
    b = layouts.scaled_config(4, max_seqs=1, max_len=1000)
    _, _, o64 = oracle_step(b)
    _, whole = gpu_step(b, partition=1024)
    _, split = gpu_step(b, partition=16)
    for name, o in (("whole", whole), ("split", split)):
        assert_decode_close(layouts.from_device(o, "f16"), o64, "f16", name)
    diff = (whole.float() - split.float()).abs().max().item()
    assert diff <= 1e-3, diff


def test_empty_context_gives_zeros():
    b = layouts.make_paged_batch(num_q_heads=4, num_kv_heads=4, head_dim=64, dtype="f16",
                                 block_size=16, context_lens=np.array([5, 40]), seed=6)
    t = layouts.to_device(b)
    t["context_lens"][0] = 0
    out = ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                     b.scale, 40, partition=16)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0)
    o64 = O.ref_decode(b.q[1:], b.k_cache, b.v_cache, b.block_tables[1:], b.context_lens[1:],
                       b.scale, "f16")
    assert_decode_close(layouts.from_device(out, "f16")[1:], o64, "f16", "after empty")


def test_out_of_range_table_entry_is_caught_in_debug_mode(monkeypatch):
    b = layouts.scaled_config(1)
    t = layouts.to_device(b)
    t["block_tables"][0, 1] = b.num_blocks + 5
    monkeypatch.setenv("PA_DEBUG", "1")
    with pytest.raises(ops.PagedAttentionError) as e:
        ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                   b.scale, b.max_context_len)
    assert e.value.code == 6
    t["slot_mapping"][0] = b.num_blocks * b.block_size
    with pytest.raises(ops.PagedAttentionError) as e:
        ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_cache"], t["v_cache"],
                              t["slot_mapping"])
    assert e.value.code == 6


def test_out_of_range_table_entries_are_clamped_without_debug_mode():
    """Without PA_DEBUG, entries outside [0, num_blocks) are clamped into the
    pool by the kernel (no read leaves it); the other sequences' outputs are
    bit-identical to a run with a clean table (the work split depends on the
    lengths only), in both forms."""
    b = layouts.scaled_config(2, poison=False, max_seqs=4, max_len=700)
    for partition in (0, 64):
        t = layouts.to_device(b)
        clean = ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                           t["context_lens"], b.scale, b.max_context_len, partition=partition)
        t["block_tables"][1, 0] = b.num_blocks + 100
        t["block_tables"][1, 2] = -7
        bad = ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                         t["context_lens"], b.scale, b.max_context_len, partition=partition)
        torch.cuda.synchronize()
        keep = [0, 2, 3]
        assert torch.equal(clean[keep].view(torch.int16), bad[keep].view(torch.int16))
        assert torch.isfinite(bad[1].float()).all()


def test_balanced_and_fixed_forms_agree():
    """The balanced single launch and fixed partitions (two launches) both meet
    the oracle, and agree with each other to float32 rounding."""
    b = layouts.scaled_config(3, max_seqs=4, max_len=700, poison=True)
    _, _, o64 = oracle_step(b)
    t = layouts.to_device(b)
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_cache"], t["v_cache"],
                          t["slot_mapping"])
    outs = {}
    for partition in (0, 64, 512):
        outs[partition] = ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                     t["context_lens"], b.scale, b.max_context_len,
                                     partition=partition)
    torch.cuda.synchronize()
    for partition, o in outs.items():
        assert_decode_close(layouts.from_device(o, "bf16"), o64, "bf16", f"P={partition}")
    diff = (outs[0].float() - outs[64].float()).abs().max().item()
    assert diff <= 8e-3, diff


def _counters(ws, num_items):
    return ws[:4 * num_items].view(torch.int32)


def test_balanced_form_reuses_its_workspace():
    """Back-to-back calls on one workspace give bit-identical outputs, and the
    arrival counters are zero again after every call (PA_DEBUG also checks
    them on entry)."""
    b = layouts.scaled_config(2, max_seqs=4, max_len=700)
    t = layouts.to_device(b)
    ws = ops.new_workspace(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                           b.max_context_len, t["q"].dtype, "cuda")
    outs = []
    for _ in range(3):
        outs.append(ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                               t["context_lens"], b.scale, b.max_context_len, workspace=ws))
        torch.cuda.synchronize()
        assert int(_counters(ws, b.num_seqs * b.num_kv_heads).abs().sum()) == 0
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_balanced_form_tiny_work_split_across_many_workgroups():
    """16 tiles of work under a max_context_len bound of 4096 (a table 256
    blocks wide): the grid is sized from the bound, so most workgroups get no
    tile and each head is split over several workgroups and combined by the
    last one. With the true bound (50) each head gets one workgroup."""
    b = layouts.make_paged_batch(num_q_heads=4, num_kv_heads=4, head_dim=64, dtype="f32",
                                 block_size=16, context_lens=[50], seed=1, poison=True,
                                 num_blocks=320, fresh_block_write=True, extra_table_cols=252)
    assert b.block_tables.shape[1] * 16 >= 4096
    _, _, o64 = oracle_step(b)
    for bound in (b.max_context_len, 4096):
        t = layouts.to_device(b, "cuda")
        ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_cache"], t["v_cache"],
                              t["slot_mapping"])
        out = ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                         t["context_lens"], b.scale, bound)
        torch.cuda.synchronize()
        assert_decode_close(layouts.from_device(out, "f32"), o64, "f32",
                            f"tiny balanced, bound {bound}")


def test_balanced_form_many_sequences_and_empty_ones():
    """600 sequences (the plan's prefix sum spans several chunks), some of
    length 0 (zero rows), then more than 4096 sequences (fixed-partition
    fallback). The step's cache write lands first (its slots start poisoned)."""
    rng = np.random.default_rng(31)
    lens = rng.integers(1, 120, size=600).astype(np.int32)
    b = layouts.make_paged_batch(num_q_heads=4, num_kv_heads=2, head_dim=64, dtype="f16",
                                 block_size=16, context_lens=lens, seed=32, poison=True)
    kc, vc, _ = oracle_step(b, seqs=[0])
    t = layouts.to_device(b)
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_cache"], t["v_cache"],
                          t["slot_mapping"])
    empty = [0, 17, 599]
    t["context_lens"][empty] = 0
    out = ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                     b.scale, b.max_context_len)
    torch.cuda.synchronize()
    keep = np.setdiff1d(np.arange(600), empty)
    o64 = O.ref_decode(b.q[keep], kc, vc, b.block_tables[keep], b.context_lens[keep], b.scale,
                       "f16")
    got = layouts.from_device(out, "f16")
    assert_decode_close(got[keep], o64, "f16", "600 seqs")
    assert not got[empty].any()

    lens = rng.integers(1, 40, size=4100).astype(np.int32)
    b = layouts.make_paged_batch(num_q_heads=1, num_kv_heads=1, head_dim=64, dtype="f16",
                                 block_size=16, context_lens=lens, seed=33, poison=True)
    _, _, o64 = oracle_step(b)
    _, out = gpu_step(b)
    assert_decode_close(layouts.from_device(out, "f16"), o64, "f16", "4100 seqs")


def test_long_rounds_and_windows():
    """Chunks of many rounds per wave and segments longer than one window
    (252 tiles for 16-token blocks, 128 for 8-token blocks), both forms."""
    for bs, hkv, lens in ((16, 2, [4100, 700, 33]), (8, 2, [2100, 515]), (32, 4, [5000, 1])):
        b = layouts.make_paged_batch(num_q_heads=2 * hkv, num_kv_heads=hkv, head_dim=128,
                                     dtype="f16", block_size=bs,
                                     context_lens=np.array(lens, np.int32), seed=40 + bs,
                                     poison=True)
        _, _, o64 = oracle_step(b)
        for partition in (0, 512, 4096):
            _, out = gpu_step(b, partition=partition)
            assert_decode_close(layouts.from_device(out, "f16"), o64, "f16",
                                f"B{bs} P={partition}")


# ---------------------------------------------------------------------------
# the fused decode step (cache write + attention in one launch)
# ---------------------------------------------------------------------------

def _two_calls(b, t):
    ops.reshape_and_cache(t["new_key"], t["new_value"], t["k_cache"], t["v_cache"],
                          t["slot_mapping"])
    return ops.decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                      b.scale, b.max_context_len)


def _fused(b, t):
    return ops.decode_step(t["q"], t["new_key"], t["new_value"], t["k_cache"], t["v_cache"],
                           t["slot_mapping"], t["block_tables"], t["context_lens"], b.scale,
                           b.max_context_len)


def _same_bits(x, y):
    if x.dtype == torch.float32:
        return torch.equal(x.view(torch.int32), y.view(torch.int32))
    return torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_decode_step_equals_write_then_decode(cfg):
    """Same pools and bit-identical output as the two separate calls; the new
    tokens' slots start poisoned, so reading them from the pools would show."""
    b = layouts.scaled_config(cfg, poison=True, max_seqs=4, max_len=700)
    _, _, o64 = oracle_step(b)
    t1 = layouts.to_device(b)
    t2 = layouts.to_device(b)
    o_sep = _two_calls(b, t1)
    o_fused = _fused(b, t2)
    torch.cuda.synchronize()
    assert _same_bits(o_sep, o_fused)
    assert _same_bits(t1["k_cache"], t2["k_cache"]) and _same_bits(t1["v_cache"], t2["v_cache"])
    assert_decode_close(layouts.from_device(o_fused, b.dtype), o64, b.dtype, f"step {b.name}")


def test_decode_step_skipped_slots_and_empty_sequences():
    """slot < 0: nothing written, the last position is read from the pool (as
    the two calls do); a sequence of length 0 still gets its write."""
    b = layouts.scaled_config(2, poison=False, max_seqs=4, max_len=300)
    t1 = layouts.to_device(b)
    t2 = layouts.to_device(b)
    for t in (t1, t2):
        t["slot_mapping"][1] = -1
        t["context_lens"][3] = 0
    o_sep = _two_calls(b, t1)
    o_fused = _fused(b, t2)
    torch.cuda.synchronize()
    assert _same_bits(o_sep, o_fused)
    assert torch.all(o_fused[3] == 0)
    assert _same_bits(t1["k_cache"], t2["k_cache"]) and _same_bits(t1["v_cache"], t2["v_cache"])


def test_decode_step_many_sequences_falls_back():
    """More than 4096 sequences: write, then fixed partitions (two launches)."""
    rng = np.random.default_rng(35)
    lens = rng.integers(1, 40, size=4100).astype(np.int32)
    b = layouts.make_paged_batch(num_q_heads=2, num_kv_heads=1, head_dim=64, dtype="f16",
                                 block_size=16, context_lens=lens, seed=36, poison=True)
    _, _, o64 = oracle_step(b)
    t = layouts.to_device(b)
    out = _fused(b, t)
    torch.cuda.synchronize()
    assert_decode_close(layouts.from_device(out, "f16"), o64, "f16", "step 4100 seqs")


def test_decode_step_checks_slots_in_debug_mode(monkeypatch):
    """A token written over a position the launch also reads (here its own
    position n - 2) breaks the step's precondition; PA_DEBUG reports it."""
    b = layouts.scaled_config(2, max_seqs=4, max_len=300)
    t = layouts.to_device(b)
    n, bs = int(b.context_lens[2]), b.block_size
    pos = n - 2
    t["slot_mapping"][2] = int(b.block_tables[2, pos // bs]) * bs + pos % bs
    monkeypatch.setenv("PA_DEBUG", "1")
    with pytest.raises(ops.PagedAttentionError) as e:
        _fused(b, t)
    assert e.value.code == 6


@pytest.mark.parametrize("debug", [False, True])
def test_decode_step_writes_outside_the_context(monkeypatch, debug):
    """A token written to a slot no sequence attends (a free block): the fused
    step writes the row and reads the sequence's last position from the pool,
    bit-identical to the two calls, with PA_DEBUG's check passing too."""
    b = layouts.scaled_config(2, poison=False, max_seqs=4, max_len=300)
    bs = b.block_size
    used = {int(b.block_tables[s, j]) for s in range(b.num_seqs)
            for j in range((int(b.context_lens[s]) + bs - 1) // bs)}
    free = next(i for i in range(b.k_cache.shape[0]) if i not in used)
    t1 = layouts.to_device(b)
    t2 = layouts.to_device(b)
    for t in (t1, t2):
        t["slot_mapping"][1] = free * bs + 3
    if debug:
        monkeypatch.setenv("PA_DEBUG", "1")
    o_sep = _two_calls(b, t1)
    o_fused = _fused(b, t2)
    torch.cuda.synchronize()
    assert _same_bits(o_sep, o_fused)
    assert _same_bits(t1["k_cache"], t2["k_cache"]) and _same_bits(t1["v_cache"], t2["v_cache"])
    row = layouts.from_device(t2["k_cache"], b.dtype)[free, :, 3]
    assert np.array_equal(row.view(np.uint8), b.new_key[1].view(np.uint8))
