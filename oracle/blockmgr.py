"""Plain model of the paged KV block manager: the CPU oracle of the C++ block manager.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU baseline
may use it; the library never does. It shares nothing with the C++ code. Lists and
dicts, no cleverness: every operation is the rule the pages state, written out.

Pages cited (titles as published):
  [P1] "vLLM 源码解析：PagedAttention 如何让大模型推理提速 10 倍"
  [P2] "vLLM 核心源码深度解析：PagedAttention 的 KV Cache 管理、Scheduler 调度引擎与
        Continuous Batching 实现全解"
  [P3] "论文专题讲解：vLLM / PagedAttention：为什么 KV cache 需要分页管理"

Rules and where they come from:
  * A block holds block_size tokens; token position p lives in logical block
    p // block_size at offset p % block_size of the sequence's block table
    ([P2] "Block 的定义", "Block Table 数据结构").
  * Free blocks sit in a free list; allocation pops one and release pushes it back,
    both O(1) ([P2] "内存分配与回收流程", and the allocate listing of "BlockAllocator
    源码核心", which pops the list). Read as a stack: the block released last is
    handed out first (reading B5); a new pool hands out `order` front to back.
  * Blocks are taken only when needed: a prompt of n tokens takes ceil(n / bs)
    blocks, a decoded token takes a new block only when the last one is full
    ([P3] "Block table：为什么它能减少碎片", [P1] section 六).
  * Shared blocks carry a reference count; a sequence that writes into a block
    whose count is above one first copies it to a new block (copy-on-write) and the
    old block's count drops by one ([P3] "共享前缀和 copy-on-write", [P1] section 五,
    [P2] "Copy-on-Write 与 Prefix Caching").
  * Prefix caching: a full block is found again by the tokens it holds, so a later
    prompt with the same prefix references it instead of taking a new block
    ([P2] "Copy-on-Write 与 Prefix Caching"). The printed hash covers only the
    block's own tokens; a block's keys and values depend on every token before it,
    so the key here is the whole token prefix up to the block's end (reading B1).
    Only full blocks are cached (reading B2).
  * When no block is free, the least recently used cold block is evicted
    ([P2] "BlockAllocator 源码核心：vLLM 的显存管理心脏", allocate: evict() when the
    free list is empty). A cold block is a cached block nobody references; it keeps
    its contents until evicted, so a prefix hit can still revive it (reading B3).
    Blocks that are not cached go straight back to the free list.
  * Capacity is checked before anything changes ([P1] section 六: can_allocate before
    admission); an operation that cannot get its blocks raises NoSpace and leaves
    the state as it was.

Readings where the pages are silent:
  B1  the cache key of logical block j is the tuple of tokens 0 .. (j+1)*bs - 1;
  B2  partial blocks are never cached; a block becomes cached when it is full;
  B3  recency is the order of release: a sequence releases its blocks from the last
      to the first, so a prompt's first blocks (the most shareable) are the last to
      be evicted; a block whose count drops to zero goes to the back of the LRU list;
  B4  the slot of a token is physical_block * block_size + offset;
  B5  the free list is a stack (pop and push at the same end).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class NoSpace(RuntimeError):
    """Neither a free nor a cold (evictable) block is left for the request."""


def blocks_for(num_tokens: int, block_size: int) -> int:
    """ceil(num_tokens / block_size)."""
    return (num_tokens + block_size - 1) // block_size


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, order: Optional[Sequence[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("num_blocks >= 0 and block_size > 0")
        order = list(range(num_blocks)) if order is None else [int(x) for x in order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of the block IDs")
        self.bs = block_size
        self.num_blocks = num_blocks
        self.free: List[int] = order[::-1]      # a stack: the end is handed out next
        self.ref: List[int] = [0] * num_blocks
        self.cold: List[int] = []               # cached, unreferenced; front = least recent
        self.cache: Dict[Tuple[int, ...], int] = {}
        self.key_of: Dict[int, Tuple[int, ...]] = {}
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}
        self.tokens: Dict[int, Optional[List[int]]] = {}

    # ------------------------------------------------------------------ blocks
    def available(self) -> int:
        return len(self.free) + len(self.cold)

    def can_allocate(self, num_tokens: int) -> bool:
        return blocks_for(num_tokens, self.bs) <= self.available()

    def _take(self) -> int:
        if self.free:
            b = self.free.pop()
        elif self.cold:
            b = self.cold.pop(0)                # the least recently released
            del self.cache[self.key_of.pop(b)]
        else:
            raise NoSpace("no free or cold block")
        self.ref[b] = 1
        return b

    def _hold(self, b: int) -> None:
        if self.ref[b] == 0:
            self.cold.remove(b)                 # a cold block revived by a prefix hit
        self.ref[b] += 1

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.cold.append(b)
            else:
                self.free.append(b)

    def _register(self, sid: int, j: int) -> None:
        """Cache full block j of sequence sid under its token prefix, if the prefix is
        not cached yet and the block is not cached under another key."""
        toks = self.tokens[sid]
        if toks is None:
            return
        key = tuple(toks[:(j + 1) * self.bs])
        b = self.tables[sid][j]
        if key not in self.cache and b not in self.key_of:
            self.cache[key] = b
            self.key_of[b] = key

    # ------------------------------------------------------------------ sequences
    def add_sequence(self, sid: int, num_tokens: int,
                     token_ids: Optional[Sequence[int]] = None) -> int:
        """Place a prompt of num_tokens tokens. With token_ids, leading full blocks whose
        prefix is cached are shared. Returns the number of prompt tokens found cached."""
        if sid in self.tables:
            raise ValueError(f"sequence {sid} exists")
        if token_ids is not None and len(token_ids) != num_tokens:
            raise ValueError("one token id per prompt token")
        hits: List[int] = []
        if token_ids is not None:
            for j in range(num_tokens // self.bs):
                b = self.cache.get(tuple(token_ids[:(j + 1) * self.bs]))
                if b is None:
                    break
                hits.append(b)
        misses = blocks_for(num_tokens, self.bs) - len(hits)
        cold_hits = sum(1 for b in hits if self.ref[b] == 0)
        if misses > len(self.free) + len(self.cold) - cold_hits:
            raise NoSpace(f"prompt needs {misses} new blocks")
        for b in hits:
            self._hold(b)
        table = hits + [self._take() for _ in range(misses)]
        self.tables[sid] = table
        self.lengths[sid] = num_tokens
        self.tokens[sid] = None if token_ids is None else [int(t) for t in token_ids]
        for j in range(len(hits), num_tokens // self.bs):
            self._register(sid, j)
        return len(hits) * self.bs

    def fork(self, parent: int, child: int) -> None:
        """child shares every block of parent (parallel sampling, beam search)."""
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        table = list(self.tables[parent])
        for b in table:
            self._hold(b)
        self.tables[child] = table
        self.lengths[child] = self.lengths[parent]
        toks = self.tokens[parent]
        self.tokens[child] = None if toks is None else list(toks)

    def append_token(self, sid: int, token_id: int = 0) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Place the next token of sid. Returns (slot, copy) where copy is the (src, dst)
        block pair to copy before the write (copy-on-write), or None."""
        table = self.tables[sid]
        pos = self.lengths[sid]
        j, off = divmod(pos, self.bs)
        fresh = j == len(table)
        shared = not fresh and self.ref[table[j]] > 1
        if (fresh or shared) and self.available() == 0:
            raise NoSpace("no block for the new token")
        copy = None
        if fresh:
            table.append(self._take())
        elif shared:
            new = self._take()
            copy = (table[j], new)
            self._release(table[j])
            table[j] = new
        self.lengths[sid] = pos + 1
        if self.tokens[sid] is not None:
            self.tokens[sid].append(int(token_id))
        if (pos + 1) % self.bs == 0:
            self._register(sid, j)
        return table[j] * self.bs + off, copy

    def free_sequence(self, sid: int) -> None:
        """Release a finished sequence's blocks, last block first (reading B3)."""
        for b in reversed(self.tables.pop(sid)):
            self._release(b)
        del self.lengths[sid]
        del self.tokens[sid]

    # ------------------------------------------------------------------ views
    def block_table(self, sid: int) -> List[int]:
        return list(self.tables[sid])

    def num_tokens(self, sid: int) -> int:
        return self.lengths[sid]

    def refcount(self, b: int) -> int:
        return self.ref[b]

    def build_tables(self, sids: Sequence[int], width: int) -> Tuple[List[List[int]], List[int]]:
        """Block tables of sids as rows of `width` entries padded with -1, and their
        context lengths."""
        rows = []
        for s in sids:
            t = self.tables[s]
            if len(t) > width:
                raise ValueError("table wider than width")
            rows.append(t + [-1] * (width - len(t)))
        return rows, [self.lengths[s] for s in sids]
