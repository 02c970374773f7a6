"""Byte and flop counts of the paged-decode path (host arithmetic only).

The benchmark divides the algorithmic byte count of one call by its measured
time to get the KV-read bandwidth; the tests check these formulas against the
sizes the pages print.

[KVP]   "PagedAttention：KV Cache 的分页革命" (openeuler.csdn.net)
[INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理" (jsqmd.com)
"""

from __future__ import annotations

from typing import Sequence

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

# MI355X published peaks used as roofline denominators.
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}


def kv_bytes_per_token_per_layer(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K plus V of one token in one layer ([INFRA] §2.1: 8 KB + 8 KB for LLaMA-7B)."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def kv_cache_bytes(num_layers: int, num_kv_heads: int, head_dim: int, num_tokens: int,
                   elem_bytes: int, batch: int = 1) -> int:
    """Whole-model KV cache of ``batch`` requests of ``num_tokens`` tokens."""
    return batch * num_layers * num_tokens * kv_bytes_per_token_per_layer(
        num_kv_heads, head_dim, elem_bytes)


def blocks_needed(num_tokens: int, block_size: int) -> int:
    return -(-num_tokens // block_size)


def page_table_bytes(max_tokens: int, block_size: int, entry_bytes: int) -> int:
    """One table covering ``max_tokens`` tokens ([KVP] page-table section)."""
    return blocks_needed(max_tokens, block_size) * entry_bytes


def block_bytes_all_layers(block_size: int, num_layers: int, num_kv_heads: int,
                           head_dim: int, elem_bytes: int) -> int:
    """One block of ``block_size`` tokens across every layer ([INFRA] §5)."""
    return block_size * num_layers * kv_bytes_per_token_per_layer(
        num_kv_heads, head_dim, elem_bytes)


def blocks_that_fit(free_bytes: int, bytes_per_block: int) -> int:
    return free_bytes // bytes_per_block


def decode_algorithmic_bytes(context_lens: Sequence[int], num_q_heads: int,
                             num_kv_heads: int, head_dim: int, elem_bytes: int,
                             block_size: int, unique_blocks: int | None = None,
                             unique_tokens: int | None = None) -> int:
    """Bytes one decode call must move.

    Each attended token's K and V row for every KV head, the queries read and
    the outputs written once, one 4-byte table entry per block attended and
    one 4-byte length per sequence. With ``unique_tokens`` the KV term counts
    each distinct cache slot once (a prefix shared by several sequences, whose
    tables name the same blocks, is read from HBM once); ``unique_blocks``
    counts whole distinct blocks instead (exact when every block is full).
    """
    num_seqs = len(context_lens)
    if unique_tokens is not None:
        kv = unique_tokens * num_kv_heads * head_dim * 2 * elem_bytes
    elif unique_blocks is None:
        kv = sum(int(n) for n in context_lens) * num_kv_heads * head_dim * 2 * elem_bytes
    else:
        kv = unique_blocks * block_size * num_kv_heads * head_dim * 2 * elem_bytes
    q_and_out = 2 * num_seqs * num_q_heads * head_dim * elem_bytes
    tables = 4 * sum(blocks_needed(int(n), block_size) for n in context_lens)
    return kv + q_and_out + tables + 4 * num_seqs


def unique_context_tokens(block_tables, context_lens: Sequence[int], block_size: int) -> int:
    """Distinct cache slots the sequences attend to: position i of sequence s
    lives in slot block_tables[s][i // B] * B + i % B, and sequences that share
    blocks ([INFRA] §4.3, copy-on-write prefix sharing) share those slots."""
    slots = set()
    for s, n in enumerate(context_lens):
        row = block_tables[s]
        for j in range(blocks_needed(int(n), block_size)):
            used = min(block_size, int(n) - j * block_size)
            base = int(row[j]) * block_size
            slots.update(range(base, base + used))
    return len(slots)


def kv_read_bytes(context_lens: Sequence[int], num_kv_heads: int, head_dim: int,
                  elem_bytes: int) -> int:
    """The K and V bytes alone (the dominant term)."""
    return sum(int(n) for n in context_lens) * num_kv_heads * head_dim * 2 * elem_bytes


def reshape_and_cache_bytes(num_tokens: int, num_kv_heads: int, head_dim: int,
                            elem_bytes: int) -> int:
    """Read key and value, write them into the pools, read the slot list."""
    return 4 * num_tokens * num_kv_heads * head_dim * elem_bytes + 4 * num_tokens


def decode_flops(context_lens: Sequence[int], num_q_heads: int, head_dim: int) -> int:
    """Multiply-adds of QK^T and PV, two flops each."""
    return 4 * sum(int(n) for n in context_lens) * num_q_heads * head_dim


def internal_fragmentation(context_lens: Sequence[int], block_size: int) -> float:
    """Share of allocated slots that hold no token: each sequence owns
    ceil(n / B) blocks and uses n of their slots ([KVP] "Block 大小的选择":
    larger blocks mean fewer table entries but more waste in the last block)."""
    used = sum(int(n) for n in context_lens)
    allocated = sum(blocks_needed(int(n), block_size) * block_size for n in context_lens)
    return 0.0 if allocated == 0 else (allocated - used) / allocated


def prefill_flops(context_lens: Sequence[int], chunk_lens: Sequence[int], num_q_heads: int,
                  head_dim: int) -> int:
    """Flops of a causal chunked prefill: a chunk of L tokens ending a context
    of n sees n - L + 1, ..., n keys per token and head; each (token, head,
    key) costs 2 * D for the score and 2 * D for the weighted value."""
    pairs = 0
    for n, chunk in zip(context_lens, chunk_lens):
        n, chunk = int(n), int(chunk)
        pairs += chunk * (n - chunk) + chunk * (chunk + 1) // 2
    return 4 * head_dim * num_q_heads * pairs


def prefill_algorithmic_bytes(context_lens: Sequence[int], chunk_lens: Sequence[int],
                              num_q_heads: int, num_kv_heads: int, head_dim: int,
                              elem_bytes: int, block_size: int) -> int:
    """Bytes a chunked prefill must move at least once: the K and V rows of
    every cached token, the queries and outputs of every chunk token, the
    table entries and the lengths and chunk starts."""
    kv = sum(int(n) for n in context_lens) * num_kv_heads * head_dim * 2 * elem_bytes
    q_and_out = 2 * sum(int(c) for c in chunk_lens) * num_q_heads * head_dim * elem_bytes
    tables = 4 * sum(blocks_needed(int(n), block_size) for n in context_lens)
    return kv + q_and_out + tables + 8 * len(context_lens) + 4
