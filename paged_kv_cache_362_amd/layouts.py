"""Seeded synthetic inputs for the paged-decode path.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic. Tests feed the same arrays to the float64 oracle and to
the HIP library, and the benchmark uses them as its workload.

Recipe (one numpy ``default_rng(seed)`` per batch, seed = config number unless
given). Draw order: context lengths, then the permutation that orders the
pool's free list, then q, the K pool, the V pool, the new tokens' K and V.
Values are float32 N(0, 1) rounded to nearest-even in the storage dtype.
Pools hold ``ceil(1.25 * blocks needed)`` blocks unless stated otherwise; the
free list hands out blocks in the permutation's order, so each request's
blocks are scattered over the pool. With ``poison=True`` every slot that no
sequence uses (unused blocks, the unused tail of a last block, table padding
entries, which point at an unused block) and every slot this step's cache write
targets holds NaN, so a kernel that reads outside the context, or attends
before the write lands, produces NaN.

The five workloads (shapes of the models the pages discuss: LLaMA-7B and
LLaMA-13B layers, [INFRA] §2.1 and [KVP]; the op example of [OPS] with 32 heads
of dim 64 and 8192 tokens in 512 blocks):

1  tiny: 1 seq, 4/4 heads, D 64, f32, n 50, B 16, pool 64, table = 4 random
   distinct blocks; the step writes the 51st token into a freshly allocated
   block (the next block on the free list).
2  LLaMA-7B layer MHA: 32 seqs, 32/32 heads, D 128, f16, B 16, n ~ U[128, 2048].
3  GQA: 64 seqs, 32/8 heads, D 128, bf16, B 16, n ~ round(LogNormal(ln 1536,
   0.5)) clipped to [64, 4096].
4  long context: 1 seq, 32/32 heads, D 64, f16, B 16, n 8192 (512 blocks).
5  LLaMA-13B layer with shared prefix: 8 seqs, 40/40 heads, D 128, f16, B 32,
   n 4096; sequences 0-3 share their first 2048 tokens (the same 64 physical
   blocks), the rest of every table is private.

For configs 2-5 the step writes one new token per sequence at position n-1
(the context length includes the token written this step).

[KVP]   "PagedAttention：KV Cache 的分页革命" (openeuler.csdn.net)
[INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理" (jsqmd.com)
[OPS]   the l189.com article on the ops-transformer PagedAttention operator
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .alloc import BlockPool, RequestTable

STORAGE_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass(frozen=True)
class ConfigSpec:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int


CONFIGS: dict[int, ConfigSpec] = {
    1: ConfigSpec("tiny single sequence", 1, 4, 4, 64, "f32", 16),
    2: ConfigSpec("LLaMA-7B-layer MHA decode", 32, 32, 32, 128, "f16", 16),
    3: ConfigSpec("GQA decode", 64, 32, 8, 128, "bf16", 16),
    4: ConfigSpec("long-context split-K decode", 1, 32, 32, 64, "f16", 16),
    5: ConfigSpec("LLaMA-13B-layer decode with shared prefix", 8, 40, 40, 128, "f16", 32),
}


@dataclass
class PagedBatch:
    """Host arrays of one decode step (storage dtypes; bf16 as uint16 bits)."""

    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q: np.ndarray                 # [S, Hq, D]
    k_cache: np.ndarray           # [N, Hkv, B, D]
    v_cache: np.ndarray           # [N, Hkv, B, D]
    block_tables: np.ndarray      # [S, M] int32
    context_lens: np.ndarray      # [S] int32
    new_key: np.ndarray           # [T, Hkv, D]
    new_value: np.ndarray         # [T, Hkv, D]
    slot_mapping: np.ndarray      # [T] int32
    scale: float
    seed: int
    poisoned: bool
    unique_blocks: int
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]


# ---------------------------------------------------------------------------
# value drawing and rounding to the storage dtype
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bit patterns, nearest-even; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    out = ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def nan_value(dtype: str):
    return np.uint16(0x7FC0) if dtype == "bf16" else STORAGE_NP[dtype](np.nan)


def draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return to_storage(rng.standard_normal(size=shape, dtype=np.float32), dtype)


# ---------------------------------------------------------------------------
# context lengths of the five workloads
# ---------------------------------------------------------------------------

def config_context_lens(config: int, rng: np.random.Generator) -> np.ndarray:
    spec = CONFIGS[config]
    if config == 1:
        lens = np.array([50])
    elif config == 2:
        lens = rng.integers(128, 2049, size=spec.num_seqs)
    elif config == 3:
        draws = rng.lognormal(mean=math.log(1536.0), sigma=0.5, size=spec.num_seqs)
        lens = np.clip(np.rint(draws), 64, 4096)
    elif config == 4:
        lens = np.array([8192])
    elif config == 5:
        lens = np.full(spec.num_seqs, 4096)
    else:
        raise ValueError(f"unknown config {config}")
    return lens.astype(np.int32)


# ---------------------------------------------------------------------------
# batch construction
# ---------------------------------------------------------------------------

def make_paged_batch(*, num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
                     block_size: int, context_lens, seed: int, poison: bool = False,
                     num_blocks: int | None = None, pool_slack: float = 0.25,
                     shared_prefix_seqs: int = 0, shared_prefix_tokens: int = 0,
                     fresh_block_write: bool = False, extra_table_cols: int = 0,
                     shuffle_pool: bool = True, poison_write_slots: bool = True,
                     rng: np.random.Generator | None = None, name: str = "") -> PagedBatch:
    """Build one decode step's inputs.

    ``context_lens`` may be an array or a callable ``rng -> array`` (so that the
    lengths are the first draw). Sequences ``0 .. shared_prefix_seqs-1`` share
    their first ``shared_prefix_tokens`` tokens (whole blocks) with sequence 0.
    With ``fresh_block_write`` the step writes a single token (the position
    after sequence 0's context) into the next free block instead of one token
    per sequence at position n-1. ``shuffle_pool=False`` hands out blocks in
    ascending order, so each request's blocks are contiguous in the pool (the
    permutation is still drawn, so every value matches the shuffled layout).
    With ``poison``, slots no sequence uses hold NaN, and so do the step's
    write slots unless ``poison_write_slots`` is False.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    lens = np.asarray(context_lens(rng) if callable(context_lens) else context_lens,
                      dtype=np.int32)
    num_seqs = int(lens.shape[0])
    if shared_prefix_tokens % block_size:
        raise ValueError("a shared prefix must be whole blocks")
    prefix_blocks = shared_prefix_tokens // block_size
    need = [-(-int(n) // block_size) for n in lens]
    distinct = sum(need)
    if shared_prefix_seqs > 1:
        distinct -= (shared_prefix_seqs - 1) * prefix_blocks
    if num_blocks is None:
        num_blocks = int(math.ceil(distinct * (1.0 + pool_slack)))
        if fresh_block_write or poison:
            num_blocks = max(num_blocks, distinct + 1)
    if num_blocks < distinct:
        raise ValueError("pool smaller than the blocks the batch needs")

    order = rng.permutation(num_blocks)
    if not shuffle_pool:
        order = np.arange(num_blocks)
    pool = BlockPool(num_blocks, order)
    tables: list[RequestTable] = []
    for s in range(num_seqs):
        t = RequestTable(pool, block_size)
        if 0 < s < shared_prefix_seqs:
            t.adopt_prefix(tables[0], prefix_blocks)
            t.append_tokens(int(lens[s]) - shared_prefix_tokens)
        else:
            t.append_tokens(int(lens[s]))
        tables.append(t)

    used = sorted({b for t in tables for b in t.blocks})
    max_blocks = max(need) + extra_table_cols
    spare = [b for b in range(num_blocks) if pool.refcount(b) == 0]
    pad_block = spare[0] if spare else 0
    block_tables = np.full((num_seqs, max_blocks), pad_block, dtype=np.int32)
    for s, t in enumerate(tables):
        block_tables[s, :len(t.blocks)] = t.blocks

    q = draw(rng, (num_seqs, num_q_heads, head_dim), dtype)
    pool_shape = (num_blocks, num_kv_heads, block_size, head_dim)
    k_cache = draw(rng, pool_shape, dtype)
    v_cache = draw(rng, pool_shape, dtype)

    if fresh_block_write:
        fresh = pool.alloc()
        slots = np.array([fresh * block_size], dtype=np.int32)
    else:
        slots = np.array([t.slot(int(lens[s]) - 1) for s, t in enumerate(tables)],
                         dtype=np.int32)
    new_key = draw(rng, (slots.shape[0], num_kv_heads, head_dim), dtype)
    new_value = draw(rng, (slots.shape[0], num_kv_heads, head_dim), dtype)

    if poison:
        live = np.zeros((num_blocks, block_size), dtype=bool)
        for s, t in enumerate(tables):
            for pos in range(int(lens[s])):
                blk = t.blocks[pos // block_size]
                live[blk, pos % block_size] = True
        if poison_write_slots:
            for slot in slots:
                live[slot // block_size, slot % block_size] = False
        dead_blk, dead_off = np.nonzero(~live)
        nv = nan_value(dtype)
        k_cache[dead_blk, :, dead_off, :] = nv
        v_cache[dead_blk, :, dead_off, :] = nv

    return PagedBatch(
        dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, q=q, k_cache=k_cache,
        v_cache=v_cache, block_tables=block_tables, context_lens=lens,
        new_key=new_key, new_value=new_value, slot_mapping=slots,
        scale=float(np.float32(1.0 / math.sqrt(head_dim))), seed=seed,
        poisoned=poison, unique_blocks=len(used), name=name,
        meta={"pad_block": pad_block, "order": order})


@dataclass
class PrefillBatch:
    """Host arrays of one multi-token (chunked-prefill) call: the paged pools
    and tables of ``paged`` (their cache already holds every chunk's K/V) and
    the packed queries of the chunks."""

    paged: PagedBatch
    q: np.ndarray                 # [T, Hq, D]
    query_start_loc: np.ndarray   # [S + 1] int32
    chunk_lens: np.ndarray        # [S] int32

    @property
    def max_query_len(self) -> int:
        return int(self.chunk_lens.max()) if self.chunk_lens.size else 0

    def __getattr__(self, name):  # pools, tables, lengths, dtype ... of the paged batch
        if name == "paged":
            raise AttributeError(name)
        return getattr(self.paged, name)


def make_prefill_batch(*, num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
                       block_size: int, context_lens, chunk_lens, seed: int,
                       poison: bool = False, **kw) -> PrefillBatch:
    """Pools and tables as ``make_paged_batch`` builds them for ``context_lens``,
    then the packed queries of chunks of ``chunk_lens[s]`` tokens ending each
    sequence's context (drawn after everything else)."""
    rng = np.random.default_rng(seed)
    paged = make_paged_batch(num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                             head_dim=head_dim, dtype=dtype, block_size=block_size,
                             context_lens=context_lens, seed=seed, poison=poison, rng=rng,
                             poison_write_slots=False, **kw)
    chunks = np.asarray(chunk_lens(paged.context_lens, rng) if callable(chunk_lens)
                        else chunk_lens, dtype=np.int32)
    if chunks.shape != paged.context_lens.shape or (chunks > paged.context_lens).any() \
            or (chunks < 0).any():
        raise ValueError("one chunk length per sequence, 0 <= chunk <= context")
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = draw(rng, (int(qsl[-1]), num_q_heads, head_dim), dtype)
    return PrefillBatch(paged=paged, q=q, query_start_loc=qsl, chunk_lens=chunks)


# Multi-token workloads: [OPS]'s example call, [1, 32, 8192, 64] in fp16 with
# 16-token blocks (512 blocks), as a whole-sequence prefill and as the last of
# four 2048-token chunks; and a LLaMA-7B layer's heads (32 x 128, fp16) over a
# 4096-token prompt.
PREFILL_WORKLOADS = {
    "llama7b_prefill_4096": dict(num_q_heads=32, num_kv_heads=32, head_dim=128, dtype="f16",
                                 block_size=16, context_lens=[4096], chunk_lens=[4096]),
    "ops_prefill_8192": dict(num_q_heads=32, num_kv_heads=32, head_dim=64, dtype="f16",
                             block_size=16, context_lens=[8192], chunk_lens=[8192]),
    "ops_chunk_2048_of_8192": dict(num_q_heads=32, num_kv_heads=32, head_dim=64, dtype="f16",
                                   block_size=16, context_lens=[8192], chunk_lens=[2048]),
}


def make_prefill_workload(name: str, seed: int = 7) -> PrefillBatch:
    return make_prefill_batch(seed=seed, name=name, **PREFILL_WORKLOADS[name])


def new_tokens_are_last(b: PagedBatch) -> bool:
    """Whether each sequence's new token is written to the slot of its last
    attended position (context_lens[s] - 1), where the fused decode step
    (pa_decode_step) takes its K/V from the new rows. The tiny workload writes
    its token into a fresh block outside the attended context instead (a slot
    the step writes and does not read)."""
    for s, n in enumerate(b.context_lens):
        n = int(n)
        slot = int(b.slot_mapping[s])
        if n < 1 or slot < 0:
            continue
        last = n - 1
        if slot != int(b.block_tables[s, last // b.block_size]) * b.block_size + last % b.block_size:
            return False
    return True


def make_config(config: int, seed: int | None = None, poison: bool = False) -> PagedBatch:
    """One of the five named workloads at full size."""
    spec = CONFIGS[config]
    seed = config if seed is None else seed
    kw = {}
    if config == 1:
        kw = dict(num_blocks=64, fresh_block_write=True)
    elif config == 4:
        kw = dict(num_blocks=640)
    elif config == 5:
        kw = dict(num_blocks=1040, shared_prefix_seqs=4, shared_prefix_tokens=2048)
    return make_paged_batch(
        num_q_heads=spec.num_q_heads, num_kv_heads=spec.num_kv_heads,
        head_dim=spec.head_dim, dtype=spec.dtype, block_size=spec.block_size,
        context_lens=lambda rng: config_context_lens(config, rng), seed=seed,
        poison=poison, name=f"config{config}: {spec.name}", **kw)


def scaled_config(config: int, seed: int | None = None, poison: bool = False,
                  max_seqs: int = 4, max_len: int = 600) -> PagedBatch:
    """A small batch with a config's head counts, dtype and block size.

    Used where the oracle must finish in seconds: at most ``max_seqs``
    sequences, lengths drawn like the config's and then capped at ``max_len``.
    """
    spec = CONFIGS[config]
    seed = config if seed is None else seed

    def lens(rng):
        full = config_context_lens(config, rng)[:max_seqs]
        return np.minimum(full, max_len)

    kw = {}
    if config == 5:
        kw = dict(shared_prefix_seqs=min(2, max_seqs), shared_prefix_tokens=spec.block_size * 4)
    return make_paged_batch(
        num_q_heads=spec.num_q_heads, num_kv_heads=spec.num_kv_heads,
        head_dim=spec.head_dim, dtype=spec.dtype, block_size=spec.block_size,
        context_lens=lens, seed=seed, poison=poison,
        name=f"config{config} scaled", **kw)


def to_torch(a: np.ndarray, dtype: str):
    """A host array in storage form as a CPU torch tensor (bf16 bit patterns
    become bfloat16)."""
    import torch

    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


def prefill_to_device(b: PrefillBatch, device="cuda"):
    """torch tensors of a prefill batch on ``device``."""
    t = to_device(b.paged, device)
    t["q"] = to_torch(b.q, b.dtype).to(device)
    import torch
    t["query_start_loc"] = torch.from_numpy(b.query_start_loc).to(device)
    return t


def to_device(batch: PagedBatch, device="cuda"):
    """torch tensors of a batch on ``device`` (bf16 bit patterns become bfloat16)."""
    import torch

    def t(a: np.ndarray, dtype: str | None = None):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    d = batch.dtype
    return {
        "q": t(batch.q, d), "k_cache": t(batch.k_cache, d), "v_cache": t(batch.v_cache, d),
        "block_tables": t(batch.block_tables), "context_lens": t(batch.context_lens),
        "new_key": t(batch.new_key, d), "new_value": t(batch.new_value, d),
        "slot_mapping": t(batch.slot_mapping),
    }


def from_device(x, dtype: str) -> np.ndarray:
    """A device tensor back to host storage (bf16 as uint16 bit patterns)."""
    import torch

    x = x.detach().to("cpu").contiguous()
    if dtype == "bf16":
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()
