"""Host-side free-list block allocator; it builds the block tables the kernels read.

This is layout tooling: it decides which physical blocks of a pool hold which
tokens, the way a block manager would, so that tests and the benchmark get
realistic scattered tables. The device code never allocates.

Pages: the runtime keeps a pool of equal blocks, hands out a free block when a
request's last block is full, records it in the request's table and returns
blocks to the pool when the request ends ([KVP] "Runtime 如何管理 KV Block";
[INFRA] §3.3, the table growing from [3, 7, 1, 12] to [3, 7, 1, 12, 5]).
Several tables may point at one physical block when requests share a prompt
prefix ([INFRA] §4.3, copy-on-write prefix sharing); a reference count keeps
such a block allocated until its last user releases it.

[KVP]   "PagedAttention：KV Cache 的分页革命" (openeuler.csdn.net)
[INFRA] "【infra之路】10-PagedAttention 与 KV Cache 管理" (jsqmd.com)
"""

from __future__ import annotations

from collections import deque
from typing import Iterable


class PoolExhausted(RuntimeError):
    """Raised when a block is requested and the pool has none free."""


class BlockPool:
    """A pool of ``num_blocks`` physical blocks handed out from a free list.

    ``order`` fixes the sequence in which free blocks are handed out (a seeded
    permutation scatters a request's blocks over the pool). Freed blocks go to
    the back of the list. A device pool and the host pool that requests are
    swapped out to are two BlockPools.
    """

    def __init__(self, num_blocks: int, order: Iterable[int] | None = None,
                 block_size_hint: int | None = None):
        if num_blocks < 0:
            raise ValueError("num_blocks must be >= 0")
        self.num_blocks = int(num_blocks)
        seq = list(range(num_blocks)) if order is None else [int(b) for b in order]
        if sorted(seq) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self._free = deque(seq)
        self._refs = [0] * num_blocks
        # Tokens per block, when known: tables refuse to move between pools
        # whose blocks differ in size.
        self.block_size_hint = block_size_hint

    @property
    def num_free(self) -> int:
        return len(self._free)

    def refcount(self, block: int) -> int:
        return self._refs[block]

    def alloc(self) -> int:
        if not self._free:
            raise PoolExhausted(f"all {self.num_blocks} blocks are in use")
        block = self._free.popleft()
        self._refs[block] = 1
        return block

    def share(self, block: int) -> int:
        """Another table starts pointing at an allocated block."""
        if self._refs[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self._refs[block] += 1
        return block

    def free(self, block: int) -> None:
        if self._refs[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self._refs[block] -= 1
        if self._refs[block] == 0:
            self._free.append(block)

    def peek_free(self) -> int:
        """The block the next ``alloc`` would return (without taking it)."""
        if not self._free:
            raise PoolExhausted(f"all {self.num_blocks} blocks are in use")
        return self._free[0]


class RequestTable:
    """The block table of one request, grown one block at a time."""

    def __init__(self, pool: BlockPool, block_size: int):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.pool = pool
        self.block_size = int(block_size)
        self.blocks: list[int] = []
        self.num_tokens = 0

    def _ensure_capacity(self, num_tokens: int) -> None:
        while len(self.blocks) * self.block_size < num_tokens:
            self.blocks.append(self.pool.alloc())

    def append_tokens(self, count: int) -> list[int]:
        """Reserve ``count`` more positions; returns their flat slots."""
        start = self.num_tokens
        self._ensure_capacity(start + count)
        self.num_tokens += count
        return [self.slot(p) for p in range(start, start + count)]

    def slot(self, position: int) -> int:
        if not 0 <= position < len(self.blocks) * self.block_size:
            raise IndexError(f"position {position} has no block")
        block = self.blocks[position // self.block_size]
        return block * self.block_size + position % self.block_size

    def adopt_prefix(self, other: "RequestTable", num_blocks: int) -> None:
        """Point this (empty) table's first blocks at ``other``'s first blocks.

        The shared blocks must be full: a later write into a shared block would
        need a private copy first.
        """
        if self.blocks:
            raise ValueError("adopt_prefix needs an empty table")
        if num_blocks > len(other.blocks) or num_blocks * self.block_size > other.num_tokens:
            raise ValueError("can only share blocks that the other table has filled")
        for b in other.blocks[:num_blocks]:
            self.blocks.append(self.pool.share(b))
        self.num_tokens = num_blocks * self.block_size

    def release(self) -> None:
        for b in self.blocks:
            self.pool.free(b)
        self.blocks = []
        self.num_tokens = 0

    def fork(self) -> "RequestTable":
        """A second table over the same blocks (a beam, or a request reusing
        this one's prompt): the table is copied, the KV data is not ([INFRA]
        §4.3, beam search sharing)."""
        other = RequestTable(self.pool, self.block_size)
        other.blocks = [self.pool.share(b) for b in self.blocks]
        other.num_tokens = self.num_tokens
        return other

    def append_cow(self) -> tuple[int, list[tuple[int, int]]]:
        """Reserve the next position, copying the last block first if another
        table shares it (copy-on-write, [INFRA] §4.3).

        Returns (slot of the new position, [(src_block, dst_block)] copies the
        device must make before anything is written to that slot). A shared
        block that is full is never written again, so only a partly filled
        shared last block is copied.
        """
        pos = self.num_tokens
        copies: list[tuple[int, int]] = []
        if pos < len(self.blocks) * self.block_size:
            last = self.blocks[-1]
            if self.pool.refcount(last) > 1:
                fresh = self.pool.alloc()
                copies.append((last, fresh))
                self.pool.free(last)
                self.blocks[-1] = fresh
        else:
            self.blocks.append(self.pool.alloc())
        self.num_tokens += 1
        return self.slot(pos), copies

    def move_to(self, target: BlockPool) -> list[tuple[int, int]]:
        """Swap this request out to ``target`` (a host pool), or back in (a
        device pool): every block gets a fresh block in ``target``, the old
        ones are released, and the table now points into ``target``
        ([INFRA] §4.3, preemption by swapping).

        Returns [(old_block, new_block)] copies the device must make before the
        old blocks are reused. Shared blocks are copied like the rest: the
        moved request keeps a private copy and the other users keep theirs.
        Raises PoolExhausted, changing nothing, if ``target`` is too small.
        """
        if target is self.pool:
            raise ValueError("the table already lives in that pool")
        if target.block_size_hint is not None and target.block_size_hint != self.block_size:
            raise ValueError("the pools hold blocks of different sizes")
        if target.num_free < len(self.blocks):
            raise PoolExhausted(f"{len(self.blocks)} blocks needed, {target.num_free} free")
        mapping = [(b, target.alloc()) for b in self.blocks]
        for b in self.blocks:
            self.pool.free(b)
        self.pool = target
        self.blocks = [new for _, new in mapping]
        return mapping
