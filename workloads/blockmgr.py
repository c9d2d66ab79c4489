"""Host-side simulation of the paged KV block manager, used only to build inputs.

This module decides *where* tokens live (which physical block, which slot); it
computes nothing of the attention itself. Tests, the benchmark and the oracle all
take their block tables and slot mappings from here.

Pages cited (titles as published):
  [P1] "vLLM 源码解析：PagedAttention 如何让大模型推理提速 10 倍"
  [P2] "vLLM 核心源码深度解析：PagedAttention 的 KV Cache 管理、Scheduler 调度引擎与
        Continuous Batching 实现全解"
  [P3] "论文专题讲解：vLLM / PagedAttention：为什么 KV cache 需要分页管理"

What follows from them:
  * A block holds a fixed number of tokens (block_size); [P2] "Block 的定义".
  * A sequence keeps a list of physical block IDs ordered by logical position; a
    token at position pos lives in logical block pos // block_size at offset
    pos % block_size; [P2] "Block Table 数据结构".
  * Free blocks sit in a free list; allocation pops, release pushes, both O(1);
    [P2] "内存分配与回收流程", [P1] section 三 (BlockAllocator).
  * Blocks are only allocated when needed: a new block is taken when the last one
    is full; [P3] "Block table：为什么它能减少碎片" (Figure 6 walk-through) and [P1]
    section 六 (one page per 16 tokens, the second page only at token 17).
  * Shared blocks carry a reference count; a write into a block whose count is
    above one first copies it to a fresh block, and the writer's table entry is
    repointed; [P3] "共享前缀和 copy-on-write", [P1] section 五, [P2]
    "Copy-on-Write 与 Prefix Caching".

Reading taken where the pages are silent: the slot of a token is encoded as
``physical_block * block_size + offset`` (a flat index into the
``[num_blocks, block_size]`` token grid of one KV head); a negative slot means
"no write".
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(RuntimeError):
    """Raised when the free list is empty (the pages evict or refuse admission)."""


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Number of blocks that hold ``num_tokens`` tokens: ceil(num_tokens / block_size)."""
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens must be >= 0 and block_size > 0")
    return -(-num_tokens // block_size)


def locate(position: int, block_size: int) -> Tuple[int, int]:
    """(logical block number, offset) of a token position; [P2] "Block Table 数据结构"."""
    if position < 0:
        raise ValueError("position must be >= 0")
    return position // block_size, position % block_size


class BlockPool:
    """Free list plus per-block reference counts over ``num_blocks`` physical blocks.

    ``order`` fixes the order in which free blocks are handed out (a shuffled
    permutation scatters a sequence's blocks over the pool). Allocation pops from
    the front of that order and a freed block goes to the back, so both are O(1).
    """

    def __init__(self, num_blocks: int, order: Optional[Sequence[int]] = None):
        if order is None:
            order = range(num_blocks)
        order = [int(x) for x in order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self._free: List[int] = list(reversed(order))  # pop() takes order[0] first
        self._ref: Dict[int, int] = {}

    def num_free(self) -> int:
        return len(self._free)

    def allocate(self, n: int) -> List[int]:
        if n > len(self._free):
            raise OutOfBlocks(f"need {n} blocks, {len(self._free)} free")
        out = [self._free.pop() for _ in range(n)]
        for b in out:
            self._ref[b] = 1
        return out

    def incref(self, block: int) -> None:
        if self._ref.get(block, 0) <= 0:
            raise ValueError(f"block {block} is not allocated")
        self._ref[block] += 1

    def decref(self, block: int) -> None:
        c = self._ref.get(block, 0)
        if c <= 0:
            raise ValueError(f"block {block} is not allocated")
        if c == 1:
            del self._ref[block]
            self._free.insert(0, block)  # back of the hand-out order
        else:
            self._ref[block] = c - 1

    def refcount(self, block: int) -> int:
        return self._ref.get(block, 0)


@dataclass
class Sequence_:
    """One sequence: its block table (physical IDs in logical order) and token count."""

    table: List[int] = field(default_factory=list)
    num_tokens: int = 0

    def copy_shared(self, pool: BlockPool) -> "Sequence_":
        """A new sequence that shares every block of this one (fork for sampling)."""
        for b in self.table:
            pool.incref(b)
        return Sequence_(table=list(self.table), num_tokens=self.num_tokens)


def prefill(pool: BlockPool, num_tokens: int, block_size: int) -> Sequence_:
    """Allocate exactly the blocks a prompt of ``num_tokens`` needs."""
    seq = Sequence_()
    seq.table = pool.allocate(blocks_needed(num_tokens, block_size))
    seq.num_tokens = num_tokens
    return seq


def slot_of(seq: Sequence_, position: int, block_size: int) -> int:
    """Flat slot of an already placed token position."""
    j, off = locate(position, block_size)
    return seq.table[j] * block_size + off


def append_token(pool: BlockPool, seq: Sequence_, block_size: int,
                 copies: Optional[List[Tuple[int, int]]] = None) -> int:
    """Place one new token at the end of ``seq`` and return its slot.

    A new physical block is taken only when the last one is full. If the block
    that receives the write is shared (refcount > 1), it is first copied to a
    fresh block: the pair (src, dst) is appended to ``copies`` (the device copy
    the caller must run before the write), the table entry is repointed and the
    old block's count drops by one.
    """
    pos = seq.num_tokens
    j, off = locate(pos, block_size)
    if j == len(seq.table):
        seq.table.extend(pool.allocate(1))
    elif j > len(seq.table):
        raise RuntimeError("block table is shorter than the token count implies")
    blk = seq.table[j]
    if pool.refcount(blk) > 1:
        new = pool.allocate(1)[0]
        if copies is None:
            raise RuntimeError("write into a shared block needs a copy list")
        copies.append((blk, new))
        pool.decref(blk)
        seq.table[j] = new
        blk = new
    seq.num_tokens = pos + 1
    return blk * block_size + off


def release(pool: BlockPool, seq: Sequence_) -> None:
    """Return every block of a finished sequence to the pool."""
    for b in seq.table:
        pool.decref(b)
    seq.table = []
    seq.num_tokens = 0


def pack_tables(seqs: Sequence[Sequence_], width: Optional[int] = None, pad: int = -1):
    """Block tables as a list of equal-length rows, padded with ``pad``."""
    w = max((len(s.table) for s in seqs), default=0) if width is None else width
    rows = []
    for s in seqs:
        if len(s.table) > w:
            raise ValueError("table wider than requested width")
        rows.append(list(s.table) + [pad] * (w - len(s.table)))
    return rows
