"""CPU oracle for decode-phase PagedAttention and the cache write that feeds it.

TEST INFRASTRUCTURE. This module is a checker, not part of the product. Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it. It shares no code, table or helper with the
HIP library under ``paged_kv_cache_362_amd/`` and imports nothing from it.

Everything here is plain numpy in float64, written as the definition of what
the method computes, one (sequence, head) at a time, with no blocking, fusion or
reordering. Pages cited (the text of three web pages on PagedAttention):

  [KVP]   "PagedAttention：KV Cache 的分页革命" (openeuler.csdn.net)
  [INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理" (jsqmd.com)
  [OPS]   the l189.com article on the ops-transformer PagedAttention operator
          for the Ascend NPU

What is computed, and where the pages fix it:

* Decode attention ([INFRA] §1.1, the per-step formula; §1.2, decode_step):
  at step t the new query of one head is dotted with every cached key of that
  head, the dot products are scaled by 1/sqrt(d), normalised by a softmax, and
  the softmax weights average the cached values.
* Paging ([INFRA] §3.2 and §3.3; [KVP] "PagedAttention 为什么出现"): the cache of
  a request lives in fixed-size physical blocks of ``block_size`` tokens; the
  request's block table maps logical block j (tokens j*B .. j*B+B-1) to a
  physical block id. The worked example in [INFRA] §3.3 (table [3, 7, 1, 12],
  block_size 16, 50 tokens) fixes that rule; tests/golden holds it.
* Attention over the table ([INFRA] §3.4): scores are formed block by block in
  table order, ONE softmax is taken over all of them, and the values are summed
  block by block with the matching slice of the weights.
* Cache write ([INFRA] §1.2, the cache append; §3.3, a new token going into the
  next slot of the request's last block): the new token's K and V rows are
  copied, unchanged, into the slot that names them.
* Block copy ([INFRA] §4.3, copy-on-write of blocks that several tables share):
  a whole physical block, every head and slot, copied unchanged.
* Multi-token (chunked-prefill) attention ([INFRA] §1.1 applied to every
  token of a chunk; [OPS] calls the operator with a whole sequence of queries,
  shape [1, 32, 8192, 64], and max_new_tokens = seq_len): each query token of
  the chunk sees exactly what it would see had the tokens been decoded one at
  a time, i.e. the cached keys up to and including its own position.

Readings taken where the pages are silent or inconsistent:

* d in 1/sqrt(d) is head_dim; the caller passes ``scale`` as float32 and the
  oracle uses float64(float32(scale)) so both sides see the same constant.
* Only the first ``context_lens[s]`` positions of a sequence are attended; the
  rest of its last block and the table entries after its last block are
  ignored ([INFRA] §3.4 reads whole blocks and never masks the partly filled
  last one; the plain reading of §1.1 attends exactly to the cached tokens).
* Grouped-query attention ([INFRA] §2.1 names 8 KV heads for 32 query heads):
  query head h reads KV head h // (Hq / Hkv) (contiguous groups).
* The softmax subtracts the maximum score first (identical in exact arithmetic).
* K and V live in two pools, each [num_blocks, num_kv_heads, block_size,
  head_dim] ([OPS] keeps the K half and the V half of a page apart).
* A slot is ``block_id * block_size + offset``; a negative slot means "write
  nothing" for that token.
* A chunk of L query tokens of a sequence whose cache holds n tokens (the
  chunk's own K/V already written) occupies positions n - L .. n - 1: the
  chunk is the newest part of the context. Query token t (position
  n - L + t) attends to positions 0 .. n - L + t (causal, the plain reading of
  the per-step formula of [INFRA] §1.1 for a token at that step). Chunks of
  all sequences are packed along one token axis, sequence s owning tokens
  query_start_loc[s] .. query_start_loc[s+1] - 1.

Storage dtypes: "f32" (numpy float32), "f16" (numpy float16) and "bf16"
(numpy uint16 holding the bfloat16 bit pattern). Every value is widened to
float64 exactly before any arithmetic.
"""

from __future__ import annotations

import numpy as np

DTYPES = ("f32", "f16", "bf16")


# ---------------------------------------------------------------------------
# storage -> float64 (exact widening)
# ---------------------------------------------------------------------------

def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to float64 exactly.

    bfloat16 is the upper half of an IEEE binary32, so its bit pattern shifted
    left by 16 is that binary32 exactly; binary16 and binary32 widen exactly by
    numpy's casts.
    """
    if dtype == "f32":
        if arr.dtype != np.float32:
            raise TypeError("f32 storage must be numpy float32")
        return arr.astype(np.float64)
    if dtype == "f16":
        if arr.dtype != np.float16:
            raise TypeError("f16 storage must be numpy float16")
        return arr.astype(np.float64)
    if dtype == "bf16":
        if arr.dtype != np.uint16:
            raise TypeError("bf16 storage must be numpy uint16 bit patterns")
        as32 = (arr.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return as32.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# block-table addressing ([INFRA] §3.3)
# ---------------------------------------------------------------------------

def logical_block_of(position: int, block_size: int) -> int:
    """Logical block that holds token ``position`` (tokens 0..B-1 are block 0)."""
    return position // block_size


def offset_in_block(position: int, block_size: int) -> int:
    """Slot of token ``position`` inside its block."""
    return position % block_size


def slot_of(table_row, position: int, block_size: int) -> int:
    """Flat slot of a token: physical block id times block_size plus offset.

    The physical block id is the table entry of the token's logical block
    ([INFRA] §3.3: logical block 0 holds tokens 0-15 and maps to physical
    block 3, and so on).
    """
    phys = int(table_row[logical_block_of(position, block_size)])
    return phys * block_size + offset_in_block(position, block_size)


def slots_of_sequence(table_row, context_len: int, block_size: int) -> list[int]:
    """Flat slots of positions 0 .. context_len-1, in logical order."""
    return [slot_of(table_row, i, block_size) for i in range(context_len)]


def kv_head_for(q_head: int, group: int) -> int:
    """KV head read by query head ``q_head`` when ``group`` query heads share one."""
    return q_head // group


# ---------------------------------------------------------------------------
# gather of one sequence's cached rows
# ---------------------------------------------------------------------------

def gather_rows(cache: np.ndarray, table_row, context_len: int, kv_head: int,
                dtype: str) -> np.ndarray:
    """The first ``context_len`` rows of one KV head, in logical order, as float64.

    cache is [num_blocks, num_kv_heads, block_size, head_dim] storage.
    """
    block_size = cache.shape[2]
    slots = slots_of_sequence(table_row, context_len, block_size)
    blocks = np.array([s // block_size for s in slots], dtype=np.int64)
    offsets = np.array([s % block_size for s in slots], dtype=np.int64)
    raw = cache[blocks, kv_head, offsets, :]
    return to_f64(raw, dtype)


# ---------------------------------------------------------------------------
# attention for one query vector ([INFRA] §1.1)
# ---------------------------------------------------------------------------

def softmax(x: np.ndarray) -> np.ndarray:
    """exp(x - max x) / sum(exp(x - max x)), float64."""
    e = np.exp(x - np.max(x))
    return e / np.sum(e)


def attend(qvec: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """One query against n cached rows: returns (weights [n], output [D])."""
    scores = scale * (keys @ qvec)
    weights = softmax(scores)
    return weights, weights @ values


def scale_as_f64(scale: float) -> float:
    """The float32 scale the kernel receives, widened to float64."""
    return float(np.float64(np.float32(scale)))


def ref_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
               block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
               dtype: str, return_probs: bool = False):
    """Decode-phase paged attention, float64.

    q            [S, Hq, D] storage
    k_cache      [N, Hkv, B, D] storage (v_cache the same)
    block_tables [S, M] int32, entries past a sequence's last block ignored
    context_lens [S] int32, each >= 1

    Returns out [S, Hq, D] float64, and with ``return_probs`` also a list
    (one entry per sequence) of [Hq, n_s] softmax weights.
    """
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = num_q_heads // num_kv_heads
    sc = scale_as_f64(scale)
    q64 = to_f64(q, dtype)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    probs = []
    for s in range(num_seqs):
        n = int(context_lens[s])
        if n < 1:
            raise ValueError("context_lens must be >= 1")
        row = block_tables[s]
        p_s = np.zeros((num_q_heads, n), dtype=np.float64)
        for kh in range(num_kv_heads):
            keys = gather_rows(k_cache, row, n, kh, dtype)
            vals = gather_rows(v_cache, row, n, kh, dtype)
            for h in range(num_q_heads):
                if kv_head_for(h, group) != kh:
                    continue
                w, o = attend(q64[s, h], keys, vals, sc)
                out[s, h] = o
                p_s[h] = w
        probs.append(p_s)
    if return_probs:
        return out, probs
    return out


def query_position(context_len: int, chunk_len: int, t: int) -> int:
    """Position in the sequence of token t of a chunk of chunk_len tokens that
    ends the sequence's context_len cached tokens."""
    return context_len - chunk_len + t


def visible_keys(position: int) -> int:
    """Number of cached positions a query at ``position`` attends to (causal:
    every position up to and including its own)."""
    return position + 1


def ref_prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                block_tables: np.ndarray, context_lens: np.ndarray,
                query_start_loc: np.ndarray, scale: float, dtype: str) -> np.ndarray:
    """Multi-token (chunked-prefill) paged attention, float64.

    q               [T, Hq, D] storage: the chunks of all sequences, packed
    query_start_loc [S + 1] int: sequence s owns tokens qsl[s] .. qsl[s+1]-1
    context_lens    [S] int: cached tokens of sequence s, chunk included
                    (chunk length <= context length)
    k_cache, v_cache, block_tables as for ``ref_decode``.

    Returns out [T, Hq, D] float64: every query token attends, head by head,
    to its sequence's cached rows up to and including its own position.
    """
    num_tokens, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = num_q_heads // num_kv_heads
    qsl = [int(x) for x in query_start_loc]
    if qsl[0] != 0 or qsl[-1] != num_tokens or any(b < a for a, b in zip(qsl, qsl[1:])):
        raise ValueError("query_start_loc must rise from 0 to the number of tokens")
    sc = scale_as_f64(scale)
    q64 = to_f64(q, dtype)
    out = np.zeros((num_tokens, num_q_heads, head_dim), dtype=np.float64)
    for s in range(len(qsl) - 1):
        n = int(context_lens[s])
        chunk = qsl[s + 1] - qsl[s]
        if chunk > n:
            raise ValueError("a chunk cannot be longer than its sequence's context")
        if chunk == 0:
            continue
        row = block_tables[s]
        for kh in range(num_kv_heads):
            keys = gather_rows(k_cache, row, n, kh, dtype)
            vals = gather_rows(v_cache, row, n, kh, dtype)
            for t in range(chunk):
                seen = visible_keys(query_position(n, chunk, t))
                for h in range(num_q_heads):
                    if kv_head_for(h, group) != kh:
                        continue
                    _, o = attend(q64[qsl[s] + t, h], keys[:seen], vals[:seen], sc)
                    out[qsl[s] + t, h] = o
    return out


def prefill_flops(context_lens, query_start_loc, num_q_heads: int, head_dim: int) -> int:
    """Multiply-adds x 2 of the two products (scores and weighted values) a
    causal chunked prefill must do: 4 * D per (query head, query token,
    visible key)."""
    total = 0
    qsl = [int(x) for x in query_start_loc]
    for s in range(len(qsl) - 1):
        n, chunk = int(context_lens[s]), qsl[s + 1] - qsl[s]
        seen = sum(visible_keys(query_position(n, chunk, t)) for t in range(chunk))
        total += 4 * head_dim * num_q_heads * seen
    return total


def ref_decode_blockloop(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                         block_tables: np.ndarray, context_lens: np.ndarray,
                         scale: float, dtype: str) -> np.ndarray:
    """Second form, after [INFRA] §3.4: two passes over the block table.

    Pass 1 walks the table in order, scores each block's keys, and concatenates
    the scores; one softmax is taken over all of them; pass 2 walks the table
    again and adds each block's values weighted by the matching slice. The
    page walks whole blocks; here only the first ``context_len`` positions
    count, so the partly filled last block contributes its used slots only.
    """
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads, block_size = k_cache.shape[1], k_cache.shape[2]
    group = num_q_heads // num_kv_heads
    sc = scale_as_f64(scale)
    q64 = to_f64(q, dtype)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        n = int(context_lens[s])
        nblocks = -(-n // block_size)
        for h in range(num_q_heads):
            kh = kv_head_for(h, group)
            scores = []
            for j in range(nblocks):
                used = min(block_size, n - j * block_size)
                kblk = to_f64(k_cache[int(block_tables[s, j]), kh, :used, :], dtype)
                scores.append(sc * (kblk @ q64[s, h]))
            weights = softmax(np.concatenate(scores))
            acc = np.zeros(head_dim, dtype=np.float64)
            offset = 0
            for j in range(nblocks):
                used = min(block_size, n - j * block_size)
                vblk = to_f64(v_cache[int(block_tables[s, j]), kh, :used, :], dtype)
                acc += weights[offset:offset + used] @ vblk
                offset += used
            out[s, h] = acc
    return out


# ---------------------------------------------------------------------------
# cache write ([INFRA] §1.2 append; §3.3 next slot)
# ---------------------------------------------------------------------------

def ref_reshape_and_cache(key: np.ndarray, value: np.ndarray, k_cache: np.ndarray,
                          v_cache: np.ndarray, slot_mapping: np.ndarray):
    """Copy each token's [Hkv, D] K and V rows into the slot that names it.

    key/value [T, Hkv, D]; k_cache/v_cache [N, Hkv, B, D] of the same storage
    dtype; slot_mapping [T] int. A negative slot writes nothing. Returns new
    arrays; the inputs are not modified. The copy is of stored values, so the
    result is bit-exact by construction.
    """
    if key.dtype != k_cache.dtype or value.dtype != v_cache.dtype:
        raise TypeError("cache write does not convert dtypes")
    block_size = k_cache.shape[2]
    k_new = k_cache.copy()
    v_new = v_cache.copy()
    for t in range(key.shape[0]):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        blk = slot // block_size
        off = slot % block_size
        k_new[blk, :, off, :] = key[t]
        v_new[blk, :, off, :] = value[t]
    return k_new, v_new


def ref_copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, block_mapping: np.ndarray):
    """Copy whole physical blocks (every KV head, every slot), K and V.

    block_mapping [P, 2] int: row (src, dst) makes block dst a copy of block
    src, the step a copy-on-write takes before a shared block is written
    ([INFRA] §4.3). Destinations are distinct and are not sources. Returns new
    arrays; the inputs are not modified. Bit-exact by construction.
    """
    k_new = k_cache.copy()
    v_new = v_cache.copy()
    for src, dst in np.asarray(block_mapping).reshape(-1, 2):
        k_new[int(dst)] = k_cache[int(src)]
        v_new[int(dst)] = v_cache[int(src)]
    return k_new, v_new


def ref_swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray,
                    dst_v: np.ndarray, block_mapping: np.ndarray):
    """Copy whole blocks from one pair of pools to another (swap out to host
    memory or back in, [INFRA] §4.3). Row (src, dst) of block_mapping makes
    block dst of the destination pools a copy of block src of the source
    pools. Returns new destination arrays; the inputs are not modified."""
    k_new = dst_k.copy()
    v_new = dst_v.copy()
    for src, dst in np.asarray(block_mapping).reshape(-1, 2):
        k_new[int(dst)] = src_k[int(src)]
        v_new[int(dst)] = src_v[int(src)]
    return k_new, v_new


# ---------------------------------------------------------------------------
# small helpers used by the tests' pins
# ---------------------------------------------------------------------------

def num_blocks_for(context_len: int, block_size: int) -> int:
    """Blocks a sequence of ``context_len`` tokens occupies (ceil division)."""
    return -(-context_len // block_size)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    Used only to judge a bfloat16 output against the float64 result. A
    bfloat16 number has 8 significant bits: with x = m * 2**e and
    0.5 <= |m| < 1, the result is round_half_even(m * 2**8) * 2**(e - 8).
    Normal range only (the judged outputs are averages of N(0,1) values).
    """
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    ax = np.where(ax == 0, np.finfo(np.float32).tiny, ax)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def nan_count(x: np.ndarray) -> int:
    return int(np.count_nonzero(np.isnan(x)))


__all__ = [
    "DTYPES", "to_f64", "logical_block_of", "offset_in_block", "slot_of",
    "slots_of_sequence", "kv_head_for", "gather_rows", "softmax", "attend",
    "scale_as_f64", "ref_decode", "ref_decode_blockloop",
    "ref_reshape_and_cache", "ref_copy_blocks", "ref_swap_blocks", "ref_prefill",
    "prefill_flops", "query_position", "visible_keys", "num_blocks_for", "bf16_round", "ulp_bf16",
    "nan_count",
]
