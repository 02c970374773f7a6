"""Pins of the float64 oracle against things other than itself (CPU only).

Each ``pin_*`` function raises AssertionError when the oracle disagrees with:
the pages' worked block-table examples (tests/golden), attention written out
by brute force on tiny inputs, a library routine (torch's scaled dot-product
attention on CPU in float64), closed forms, and invariants the method must
hold. ``test_planted_mistakes_are_caught`` plants plausible mistakes in the
oracle (on the CPU) and checks that at least one pin fails for each.

[KVP]   "PagedAttention：KV Cache 的分页革命" (openeuler.csdn.net)
[INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理" (jsqmd.com)
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.paged_attention as O
from paged_kv_cache_362_amd import layouts

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# helpers that build tiny pools by hand (independent of layouts.py)
# ---------------------------------------------------------------------------

def _scatter_dense(dense_k, dense_v, tables, block_size, num_blocks, fill=0.0):
    """Place contiguous per-sequence rows into a pool following the tables.

    dense_k[s] is [n_s, Hkv, D] float32; row i goes to block tables[s][i // B]
    at offset i % B (the rule the golden worked example pins).
    """
    hkv, d = dense_k[0].shape[1], dense_k[0].shape[2]
    kc = np.full((num_blocks, hkv, block_size, d), fill, dtype=np.float32)
    vc = np.full((num_blocks, hkv, block_size, d), fill, dtype=np.float32)
    for s, (k, v) in enumerate(zip(dense_k, dense_v)):
        for i in range(k.shape[0]):
            kc[tables[s][i // block_size], :, i % block_size, :] = k[i]
            vc[tables[s][i // block_size], :, i % block_size, :] = v[i]
    return kc, vc


def _tables_array(tables, width):
    out = np.zeros((len(tables), width), dtype=np.int32)
    for s, t in enumerate(tables):
        out[s, :len(t)] = t
    return out


def _brute_force_attention(qv, keys, vals, scale):
    """Attention for one query with Python floats and math.exp."""
    n, d = len(keys), len(qv)
    scores = [scale * sum(float(qv[j]) * float(keys[i][j]) for j in range(d)) for i in range(n)]
    top = max(scores)
    w = [math.exp(x - top) for x in scores]
    z = sum(w)
    return [sum(w[i] * float(vals[i][j]) for i in range(n)) / z for j in range(d)]


def _random_case(rng, num_seqs, hq, hkv, d, block_size, lens, extra_blocks=3):
    need = [-(-n // block_size) for n in lens]
    num_blocks = sum(need) + extra_blocks
    perm = rng.permutation(num_blocks)
    tables, k = [], 0
    for nb in need:
        tables.append([int(b) for b in perm[k:k + nb]])
        k += nb
    dense_k = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
    dense_v = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
    q = rng.standard_normal((num_seqs, hq, d)).astype(np.float32)
    kc, vc = _scatter_dense(dense_k, dense_v, tables, block_size, num_blocks, fill=np.nan)
    return q, kc, vc, _tables_array(tables, max(need) + 1), np.array(lens, np.int32), dense_k, dense_v


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_worked_example_slots():
    g = _load("worked_example_block_table.json")
    expect = []
    for lo, hi, slo, shi in g["slot_ranges"]:
        assert hi - lo == shi - slo
        expect += list(range(slo, shi + 1))
    got = O.slots_of_sequence(g["table"], g["context_len"], g["block_size"])
    assert got == expect, (got, expect)
    a = g["append"]
    assert O.slot_of(a["table"], a["position"], g["block_size"]) == a["slot"]
    p = g["position_50"]
    assert O.slot_of(g["table"], p["position"], g["block_size"]) == p["slot"]


def pin_page_table_example():
    g = _load("page_table_example.json")
    got = [O.slot_of(g["table"], j * g["block_size"], g["block_size"])
           for j in range(len(g["table"]))]
    assert got == g["first_slot_of_each_block"]


def pin_ops_block_count():
    g = _load("page_figures.json")["ops_example"]
    assert O.num_blocks_for(g["tokens"], g["block_size"]) == g["blocks"]


def pin_brute_force_tiny():
    rng = np.random.default_rng(11)
    for hq, hkv, d, bs, lens in [(2, 2, 8, 4, [7, 1, 12]), (4, 2, 6, 8, [9, 17]),
                                 (3, 1, 5, 16, [33]), (2, 2, 4, 2, [5, 6])]:
        q, kc, vc, bt, cl, dk, dv = _random_case(rng, len(lens), hq, hkv, d, bs, lens)
        scale = 1.0 / math.sqrt(d)
        got = O.ref_decode(q, kc, vc, bt, cl, scale, "f32")
        sc = float(np.float32(scale))
        g = hq // hkv
        for s, n in enumerate(lens):
            for h in range(hq):
                kh = h // g
                ref = _brute_force_attention(q[s, h], dk[s][:, kh, :], dv[s][:, kh, :], sc)
                np.testing.assert_allclose(got[s, h], ref, rtol=0, atol=1e-12)


def pin_torch_sdpa_fp64():
    rng = np.random.default_rng(12)
    lens = [50, 3, 130]
    hq, hkv, d, bs = 8, 2, 64, 16
    q, kc, vc, bt, cl, dk, dv = _random_case(rng, len(lens), hq, hkv, d, bs, lens)
    scale = 1.0 / math.sqrt(d)
    got = O.ref_decode(q, kc, vc, bt, cl, scale, "f32")
    sc = float(np.float32(scale))
    for s, n in enumerate(lens):
        kk = torch.from_numpy(dk[s].astype(np.float64)).permute(1, 0, 2)  # [Hkv, n, D]
        vv = torch.from_numpy(dv[s].astype(np.float64)).permute(1, 0, 2)
        kk = kk.repeat_interleave(hq // hkv, dim=0).unsqueeze(0).contiguous()
        vv = vv.repeat_interleave(hq // hkv, dim=0).unsqueeze(0).contiguous()
        qq = torch.from_numpy(q[s].astype(np.float64)).reshape(1, hq, 1, d)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=sc)
        np.testing.assert_allclose(got[s], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)


def pin_single_token_returns_its_value():
    rng = np.random.default_rng(13)
    q, kc, vc, bt, cl, dk, dv = _random_case(rng, 2, 4, 4, 16, 8, [1, 1])
    got = O.ref_decode(q, kc, vc, bt, cl, 0.25, "f32")
    for s in range(2):
        for h in range(4):
            assert np.array_equal(got[s, h], dv[s][0, h].astype(np.float64))


def pin_zero_query_averages_values():
    rng = np.random.default_rng(14)
    q, kc, vc, bt, cl, dk, dv = _random_case(rng, 2, 2, 2, 8, 4, [13, 6])
    q[:] = 0
    got = O.ref_decode(q, kc, vc, bt, cl, 0.3, "f32")
    for s in range(2):
        for h in range(2):
            np.testing.assert_allclose(got[s, h], dv[s][:, h].astype(np.float64).mean(0),
                                       rtol=0, atol=1e-14)


def pin_identical_keys_average_values():
    rng = np.random.default_rng(15)
    q, kc, vc, bt, cl, dk, dv = _random_case(rng, 1, 2, 1, 8, 4, [11])
    row = rng.standard_normal(8).astype(np.float32)
    dk = [np.broadcast_to(row, (11, 1, 8)).copy()]
    kc, vc = _scatter_dense(dk, dv, [list(bt[0, :3])], 4, kc.shape[0], fill=np.nan)
    got = O.ref_decode(q, kc, vc, bt, cl, 0.7, "f32")
    for h in range(2):
        np.testing.assert_allclose(got[0, h], dv[0][:, 0].astype(np.float64).mean(0),
                                   rtol=0, atol=1e-14)


def pin_constant_values_give_constant_output():
    rng = np.random.default_rng(16)
    q, kc, vc, bt, cl, dk, dv = _random_case(rng, 3, 4, 2, 8, 4, [9, 1, 15])
    live = ~np.isnan(vc)
    vc[live] = 1.0
    got = O.ref_decode(q, kc, vc, bt, cl, 0.35, "f32")
    np.testing.assert_allclose(got, 1.0, rtol=0, atol=1e-14)


def _geometric_case(n=50, d=64, bs=16, a=2.0, hq=1):
    """q = a*e0, K[i] = i*e0, V[i] = e_i: weights and output in closed form."""
    k = np.zeros((n, 1, d), np.float32)
    k[:, 0, 0] = np.arange(n, dtype=np.float32)
    v = np.zeros((n, 1, d), np.float32)
    v[np.arange(n), 0, np.arange(n)] = 1.0
    q = np.zeros((1, hq, d), np.float32)
    q[0, :, 0] = a
    table = [9, 2, 30, 17, 5][: -(-n // bs)]
    kc, vc = _scatter_dense([k], [v], [table], bs, 32, fill=7.0)
    return q, kc, vc, _tables_array([table], len(table) + 2), np.array([n], np.int32)


def pin_geometric_closed_form():
    n, d, bs = 50, 64, 16
    scale = 0.125
    q, kc, vc, bt, cl = _geometric_case(n, d, bs)
    bt[0, len([9, 2, 30, 17]):] = 31  # padding entries point at a filled block
    got, probs = O.ref_decode(q, kc, vc, bt, cl, scale, "f32", return_probs=True)
    r = math.exp(float(np.float32(scale)) * 2.0)
    expect = np.array([r ** i * (1 - r) / (1 - r ** n) for i in range(n)])
    np.testing.assert_allclose(probs[0][0], expect, rtol=1e-12, atol=0)
    np.testing.assert_allclose(got[0, 0, :n], expect, rtol=1e-12, atol=0)
    assert np.all(got[0, 0, n:] == 0.0)


def pin_gqa_head_mapping():
    rng = np.random.default_rng(17)
    hq, hkv = 8, 2
    q, kc, vc, bt, cl, dk, dv = _random_case(rng, 2, hq, hkv, 8, 4, [10, 5])
    live = ~np.isnan(vc)
    for kh in range(hkv):
        vc[:, kh][live[:, kh]] = float(kh + 1)
    got = O.ref_decode(q, kc, vc, bt, cl, 0.5, "f32")
    for h in range(hq):
        np.testing.assert_allclose(got[:, h], float(h // (hq // hkv) + 1), atol=1e-14, rtol=0)


def pin_weights_sum_to_one():
    b = layouts.scaled_config(3, max_seqs=3, max_len=300)
    _, probs = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                            b.scale, b.dtype, return_probs=True)
    for p in probs:
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def pin_block_permutation_invariance():
    b = layouts.scaled_config(2, max_seqs=3, max_len=200)
    base = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                        b.scale, b.dtype)
    perm = np.random.default_rng(18).permutation(b.num_blocks)
    kc = np.empty_like(b.k_cache)
    vc = np.empty_like(b.v_cache)
    kc[perm] = b.k_cache
    vc[perm] = b.v_cache
    bt = perm[b.block_tables].astype(np.int32)
    moved = O.ref_decode(b.q, kc, vc, bt, b.context_lens, b.scale, b.dtype)
    assert np.array_equal(base, moved)


def pin_poisoned_slots_ignored():
    b = layouts.scaled_config(1, poison=True)
    clean = layouts.scaled_config(1, poison=False)
    assert np.isnan(b.k_cache).any()
    outs = []
    for x in (b, clean):
        kc, vc = O.ref_reshape_and_cache(x.new_key, x.new_value, x.k_cache, x.v_cache,
                                         x.slot_mapping)
        outs.append(O.ref_decode(x.q, kc, vc, x.block_tables, x.context_lens, x.scale, x.dtype))
    # the step's target slot is poisoned until the write lands
    stale = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                         b.scale, b.dtype)
    assert O.nan_count(stale) > 0
    assert O.nan_count(outs[0]) == 0
    assert np.array_equal(outs[0], outs[1])


def pin_gqa_equals_repeated_mha():
    b = layouts.scaled_config(3, max_seqs=2, max_len=100)
    g = b.num_q_heads // b.num_kv_heads
    o_gqa = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                         b.scale, b.dtype)
    kc = np.repeat(b.k_cache, g, axis=1)
    vc = np.repeat(b.v_cache, g, axis=1)
    o_mha = O.ref_decode(b.q, kc, vc, b.block_tables, b.context_lens, b.scale, b.dtype)
    assert np.array_equal(o_gqa, o_mha)


def pin_shared_prefix_equals_copied_prefix():
    b = layouts.scaled_config(5, max_seqs=3, max_len=300)
    base = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                        b.scale, b.dtype)
    # give sequence 1 private copies of the blocks it shares with sequence 0
    shared = [int(x) for x in b.block_tables[1] if x in set(b.block_tables[0].tolist())]
    assert shared, "scaled config 5 must share a prefix"
    extra = len(shared)
    kc = np.concatenate([b.k_cache, b.k_cache[shared]], axis=0)
    vc = np.concatenate([b.v_cache, b.v_cache[shared]], axis=0)
    bt = b.block_tables.copy()
    remap = {blk: b.num_blocks + i for i, blk in enumerate(shared)}
    bt[1] = [remap.get(int(x), int(x)) for x in bt[1]]
    assert extra > 0
    copied = O.ref_decode(b.q, kc, vc, bt, b.context_lens, b.scale, b.dtype)
    assert np.array_equal(base, copied)


def pin_blockloop_form_agrees():
    for cfg in (1, 3, 5):
        b = layouts.scaled_config(cfg, max_seqs=2, max_len=150)
        o1 = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                          b.scale, b.dtype)
        o2 = O.ref_decode_blockloop(b.q, b.k_cache, b.v_cache, b.block_tables,
                                    b.context_lens, b.scale, b.dtype)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)


def pin_cache_write_worked_example():
    g = _load("worked_example_block_table.json")
    bs, table = g["block_size"], g["table"]
    pos = g["position_50"]["position"]
    kc = np.zeros((16, 2, bs, 4), np.float16)
    vc = np.zeros((16, 2, bs, 4), np.float16)
    key = np.arange(8, dtype=np.float16).reshape(1, 2, 4) + 1
    val = -key
    slot = O.slot_of(table, pos, bs)
    k2, v2 = O.ref_reshape_and_cache(key, val, kc, vc, np.array([slot, -1], np.int32)[:1])
    assert np.array_equal(k2[12, :, 2, :], key[0]) and np.array_equal(v2[12, :, 2, :], val[0])
    k2[12, :, 2, :] = 0
    v2[12, :, 2, :] = 0
    assert not k2.any() and not v2.any()
    k3, _ = O.ref_reshape_and_cache(key, val, kc, vc, np.array([-1], np.int32))
    assert not k3.any()


def pin_bf16_widening():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F80], np.uint16)
    assert list(O.to_f64(bits, "bf16")) == [1.0, -1.0, 3.140625, 0.0, float("inf")]
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5])
    assert list(O.bf16_round(x)) == [1.0, 1.0 + 2 ** -6, 1.0, -2.5]


def _bf16_value_of_bits(bits):
    """Value of bfloat16 bit patterns, through float32: a bfloat16 number is the
    upper half of the float32 with the same sign, exponent and top mantissa bits."""
    return (np.asarray(bits, np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def pin_bf16_spacing():
    """ulp_bf16 is the gap to the next bfloat16 number, taken from bit patterns.

    For a positive bfloat16 value x with bits b (and b + 1 in the same binade
    or the first of the next), the spacing at x is value(b + 1) - value(b).
    It decides how far a bfloat16 output of magnitude >= 1 may sit from the
    rounded float64 result, so an exponent off by one would halve or double
    that bound."""
    xs = np.array([0.5, 0.75, 1.0, 1.5, 1.9921875, 2.0, 3.0, 3.890625, 7.5, 0.125])
    bits = (xs.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint32)
    assert np.array_equal(_bf16_value_of_bits(bits), xs)  # all are bfloat16 values
    gap = _bf16_value_of_bits(bits + 1) - _bf16_value_of_bits(bits)
    assert np.array_equal(O.ulp_bf16(xs), gap)
    assert np.array_equal(O.ulp_bf16(-xs), gap)  # the spacing depends on |x| only
    # closed forms: 8 significant bits, so 2**-7 on [1, 2) and 2**-6 on [2, 4)
    assert list(O.ulp_bf16(np.array([1.0, 1.9921875, 2.0, -3.0, 0.5]))) == [
        2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -8]


def pin_bf16_round_matches_library():
    """bf16_round agrees with torch's float32 -> bfloat16 conversion (round to
    nearest, ties to even) on float32 inputs, ties included."""
    rng = np.random.default_rng(11)
    x32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-6, 6, 20000))).astype(np.float32)
    # exact ties: a bfloat16 value plus half its spacing
    base = _bf16_value_of_bits(rng.integers(0x3C00, 0x4400, 2000).astype(np.uint32))
    ties = (base + O.ulp_bf16(base) / 2).astype(np.float32)
    x = np.concatenate([x32, ties, -ties]).astype(np.float64)
    lib = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(x), lib)


# --- multi-token (chunked-prefill) attention --------------------------------

def _prefill_case(rng, hq, hkv, d, bs, lens, chunks):
    """Random pools plus packed queries: sequence s has a chunk of chunks[s]
    query tokens ending its lens[s] cached tokens."""
    _, kc, vc, bt, cl, dk, dv = _random_case(rng, len(lens), hq, hkv, d, bs, lens)
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), hq, d)).astype(np.float32)
    return q, kc, vc, bt, cl, qsl, dk, dv


def pin_prefill_matches_library_attention():
    """A library routine: torch's scaled_dot_product_attention (CPU, float64)
    over the contiguous rows, with an explicit causal mask offset so that the
    chunk's queries sit at the end of the context."""
    rng = np.random.default_rng(31)
    for hq, hkv, d, bs, lens, chunks in [(4, 2, 8, 4, [13, 9], [5, 9]),
                                         (2, 2, 16, 8, [40, 3, 17], [40, 1, 6]),
                                         (6, 3, 4, 2, [11], [7])]:
        q, kc, vc, bt, cl, qsl, dk, dv = _prefill_case(rng, hq, hkv, d, bs, lens, chunks)
        scale = 1.0 / math.sqrt(d)
        got = O.ref_prefill(q, kc, vc, bt, cl, qsl, scale, "f32")
        g = hq // hkv
        for s, (n, c) in enumerate(zip(lens, chunks)):
            qs = torch.from_numpy(q[qsl[s]:qsl[s + 1]].astype(np.float64)).transpose(0, 1)
            ks = torch.from_numpy(dk[s].astype(np.float64)).transpose(0, 1)
            vs = torch.from_numpy(dv[s].astype(np.float64)).transpose(0, 1)
            ks = ks.repeat_interleave(g, dim=0)
            vs = vs.repeat_interleave(g, dim=0)
            allowed = torch.arange(n)[None, :] <= (n - c + torch.arange(c))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qs, ks, vs, attn_mask=allowed, scale=float(np.float32(scale)))
            np.testing.assert_allclose(got[qsl[s]:qsl[s + 1]],
                                       ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


def pin_prefill_single_token_chunks_are_decode():
    """Special case: chunks of one token are decode steps."""
    b = layouts.scaled_config(3, max_seqs=4, max_len=300)
    qsl = np.arange(b.num_seqs + 1, dtype=np.int32)
    got = O.ref_prefill(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, qsl,
                        b.scale, b.dtype)
    want = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale,
                        b.dtype)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def pin_prefill_first_token_is_its_value_row():
    """Closed form: the first token of a whole-sequence prefill sees only
    itself, so its output is its own V row, exactly."""
    rng = np.random.default_rng(32)
    q, kc, vc, bt, cl, qsl, dk, dv = _prefill_case(rng, 4, 4, 8, 4, [9, 6], [9, 6])
    got = O.ref_prefill(q, kc, vc, bt, cl, qsl, 0.3, "f32")
    for s in range(2):
        for h in range(4):
            assert np.array_equal(got[qsl[s], h], dv[s][0, h].astype(np.float64))


def pin_prefill_chunking_invariance():
    """Prefilling a sequence in two chunks gives the rows of one whole prefill,
    and keys after a query's position never change its output."""
    rng = np.random.default_rng(33)
    n, a = 29, 12
    q, kc, vc, bt, cl, qsl, dk, dv = _prefill_case(rng, 4, 2, 8, 4, [n], [n])
    whole = O.ref_prefill(q, kc, vc, bt, cl, qsl, 0.35, "f32")
    first = O.ref_prefill(q[:a], kc, vc, bt, np.array([a]), np.array([0, a]), 0.35, "f32")
    second = O.ref_prefill(q[a:], kc, vc, bt, cl, np.array([0, n - a]), 0.35, "f32")
    assert np.array_equal(np.concatenate([first, second]), whole)
    # overwrite the rows after position 20 with other values
    kc2, vc2 = kc.copy(), vc.copy()
    for i in range(21, n):
        kc2[bt[0, i // 4], :, i % 4] = 7.0
        vc2[bt[0, i // 4], :, i % 4] = -3.0
    moved = O.ref_prefill(q, kc2, vc2, bt, cl, qsl, 0.35, "f32")
    assert np.array_equal(moved[:21], whole[:21])
    assert not np.allclose(moved[21:], whole[21:])


def pin_prefill_flop_count():
    """Closed form: a whole-sequence causal prefill of n tokens sees
    n(n+1)/2 (query, key) pairs; [OPS]'s [1, 32, 8192, 64] call does
    4 * 64 * 32 * 8192 * 8193 / 2 flops."""
    assert O.prefill_flops([8192], [0, 8192], 32, 64) == 4 * 64 * 32 * 8192 * 8193 // 2
    # a chunk of 3 after 5 cached tokens: positions 5, 6, 7 see 6 + 7 + 8 keys
    assert O.prefill_flops([8], [0, 3], 1, 1) == 4 * (6 + 7 + 8)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _wrong_softmax_sign(x):
    e = np.exp(-(x - np.max(x)))
    return e / e.sum()


def _unnormalised_softmax(x):
    return np.exp(x - np.max(x))


def _keys_and_values_swapped(qvec, keys, values, scale):
    w = O.softmax(scale * (values @ qvec))
    return w, w @ keys


def _scale_squared(scale):
    return float(np.float32(scale)) ** 2


def _reversed_offsets(position, block_size):
    return block_size - 1 - position % block_size


def _next_logical_block(position, block_size):
    return (position + 1) // block_size


def _interleaved_groups(q_head, group):
    return q_head % 2


def _right_aligned_gather(cache, table_row, context_len, kv_head, dtype):
    """Reads the last n slots of the sequence's whole blocks instead of the first n."""
    bs = cache.shape[2]
    end = -(-context_len // bs) * bs
    pos = range(end - context_len, end)
    blocks = [int(table_row[i // bs]) for i in pos]
    offs = [i % bs for i in pos]
    return O.to_f64(cache[blocks, kv_head, offs, :], dtype)


def _ulp_exponent_off_by_one(x):
    ax = np.abs(np.asarray(x, dtype=np.float64))
    return np.exp2(np.floor(np.log2(ax)) - 6)


def _bf16_round_seven_bits(x):
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(np.ldexp(m, 7)), e - 7)


def _chunk_at_start(context_len, chunk_len, t):
    return t


def _causal_off_by_one(position):
    return position


def _causal_one_too_many(position):
    return position + 2


MUTANTS = {
    "bf16_spacing_exponent_off_by_one": ("ulp_bf16", _ulp_exponent_off_by_one),
    "bf16_round_seven_bits": ("bf16_round", _bf16_round_seven_bits),
    "prefill_chunk_at_start": ("query_position", _chunk_at_start),
    "prefill_excludes_own_key": ("visible_keys", _causal_off_by_one),
    "prefill_sees_next_key": ("visible_keys", _causal_one_too_many),
    "softmax_sign": ("softmax", _wrong_softmax_sign),
    "softmax_unnormalised": ("softmax", _unnormalised_softmax),
    "k_v_swapped": ("attend", _keys_and_values_swapped),
    "scale_squared": ("scale_as_f64", _scale_squared),
    "offset_reversed": ("offset_in_block", _reversed_offsets),
    "logical_block_shifted": ("logical_block_of", _next_logical_block),
    "gqa_interleaved": ("kv_head_for", _interleaved_groups),
    "context_window_shifted": ("gather_rows", _right_aligned_gather),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # AssertionError or an index error the mistake causes
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mutant}"


def test_copy_blocks_oracle():
    """Block copy: destination blocks equal their sources byte for byte, every
    other block is untouched, the inputs are not modified."""
    rng = np.random.default_rng(12)
    kc = rng.standard_normal((6, 2, 4, 8)).astype(np.float16)
    vc = rng.standard_normal((6, 2, 4, 8)).astype(np.float16)
    k2, v2 = O.ref_copy_blocks(kc, vc, np.array([[1, 4], [0, 5]]))
    assert np.array_equal(k2[4].view(np.int16), kc[1].view(np.int16))
    assert np.array_equal(v2[5].view(np.int16), vc[0].view(np.int16))
    for b in (0, 1, 2, 3):
        assert np.array_equal(k2[b].view(np.int16), kc[b].view(np.int16))
    assert not np.array_equal(k2[4], kc[4])


def test_swap_out_and_back_in_preserves_attention():
    """[INFRA] §4.3: a preempted request's blocks go to host memory and come
    back, usually to other device blocks; only its table changes. Attention
    over the moved-back blocks through the new table equals attention before
    the swap, exactly, and the host pool holds the blocks bit for bit."""
    b = layouts.scaled_config(2, max_seqs=3, max_len=200)
    base = O.ref_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                        b.scale, b.dtype)
    rng = np.random.default_rng(19)
    used = sorted({int(x) for row, n in zip(b.block_tables, b.context_lens)
                   for x in row[:O.num_blocks_for(int(n), b.block_size)]})
    host_k = np.zeros((len(used) + 3,) + b.k_cache.shape[1:], b.k_cache.dtype)
    host_v = np.zeros_like(host_k)
    host_of = dict(zip(used, rng.permutation(len(host_k))[:len(used)]))
    out_map = np.array(sorted(host_of.items()), np.int32)
    host_k, host_v = O.ref_swap_blocks(b.k_cache, b.v_cache, host_k, host_v, out_map)
    for dev, host in host_of.items():
        assert np.array_equal(host_k[host].view(np.uint8), b.k_cache[dev].view(np.uint8))
        assert np.array_equal(host_v[host].view(np.uint8), b.v_cache[dev].view(np.uint8))
    # back in, to a different device placement, over a cleared device pool
    back_of = dict(zip(used, rng.permutation(b.num_blocks)[:len(used)]))
    in_map = np.array([(host_of[u], back_of[u]) for u in used], np.int32)
    dev_k = np.full_like(b.k_cache, np.nan)
    dev_v = np.full_like(b.v_cache, np.nan)
    dev_k, dev_v = O.ref_swap_blocks(host_k, host_v, dev_k, dev_v, in_map)
    bt = b.block_tables.copy()
    for i, n in enumerate(b.context_lens):
        nb = O.num_blocks_for(int(n), b.block_size)
        bt[i, :nb] = [back_of[int(x)] for x in b.block_tables[i, :nb]]
    moved = O.ref_decode(b.q, dev_k, dev_v, bt, b.context_lens, b.scale, b.dtype)
    assert np.array_equal(base, moved)
