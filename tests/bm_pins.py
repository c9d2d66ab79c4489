"""Pins of the block-manager oracle (oracle/blockmgr.py) to the pages' examples and to
invariants. Each ``pin_*`` takes the BlockManager class to check (the oracle's, or a
deliberately broken subclass in tests/test_bm_oracle.py) and raises AssertionError when
it disagrees. Expected values are written by hand from the rules cited in the oracle's
header, not computed by any code in this repository.
"""
from __future__ import annotations

import json
import os
import random

from oracle.blockmgr import NoSpace

# exceptions that mean "no block left" for the class under test (the oracle's, and the
# library's when tests/test_block_manager.py runs the pins on the C++ manager)
NOSPACE = (NoSpace,)


def _exists(bm, sid):
    try:
        bm.num_tokens(sid)
        return True
    except Exception:
        return False

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pin_worked_example(BM):
    """[P3] "Block table：为什么它能减少碎片" (Figure 6) with the placement of [P1]
    section 三: bs 4, a 7-token prompt in blocks 5 and 3 (4 + 3 tokens, one free slot);
    the 8th token goes to slot 15, the 9th takes block 8 at slot 32."""
    g = _golden("worked_example_fig6.json")
    bs, order = g["block_size"], g["physical_order"]
    bm = BM(9, bs, order + [b for b in range(9) if b not in order])
    bm.add_sequence(0, g["prompt_tokens"])
    e = g["expect"]
    assert bm.block_table(0) == e["table_after_prompt"]
    assert len(bm.block_table(0)) == e["logical_blocks_after_prompt"]
    assert len(bm.block_table(0)) * bs - g["prompt_tokens"] == e["free_slots_in_last_block"]
    for d in e["decodes"]:
        slot, copy = bm.append_token(0)
        assert slot == d["slot"] and copy is None
        assert bm.block_table(0) == d["table_after"]


def pin_allocation_on_demand(BM):
    """[P1] section 六: 16-token pages; a request holds one page at its 5th and 16th
    token and a second only from its 17th, whether placed at once or token by token."""
    g = _golden("allocation_on_demand.json")
    bs = g["block_size"]
    for c in g["cases"]:
        bm = BM(8, bs)
        bm.add_sequence(0, c["tokens"])
        assert len(bm.block_table(0)) == c["pages"], c
        bm2 = BM(8, bs)
        bm2.add_sequence(0, 0)
        for _ in range(c["tokens"]):
            bm2.append_token(0)
        assert len(bm2.block_table(0)) == c["pages"], c


def pin_copy_on_write(BM):
    """[P3] "共享前缀和 copy-on-write", [P1] section 五: a forked sequence shares its
    parent's blocks (counts 2); the first writer into the shared partial block copies
    it to a fresh block and drops the old block's count; the other then writes in place.
    A block shared by 8 samples is copied by 7 writers and its count falls from 8 to 1."""
    bm = BM(10, 4)
    bm.add_sequence(0, 6)                       # blocks 0, 1 (1 holds 2 tokens)
    bm.fork(0, 1)
    assert bm.block_table(1) == [0, 1] and bm.refcount(0) == 2 and bm.refcount(1) == 2
    slot, copy = bm.append_token(1)
    assert copy == (1, 2) and slot == 2 * 4 + 2 and bm.block_table(1) == [0, 2]
    assert bm.refcount(1) == 1 and bm.refcount(2) == 1 and bm.refcount(0) == 2
    slot, copy = bm.append_token(0)
    assert copy is None and slot == 1 * 4 + 2 and bm.block_table(0) == [0, 1]
    bm = BM(16, 4)
    bm.add_sequence(0, 5)                       # blocks 0, 1
    for s in range(1, 8):
        bm.fork(0, s)
    assert bm.refcount(1) == 8
    for s in range(1, 8):
        _, copy = bm.append_token(s)
        assert copy is not None and copy[0] == 1
    assert bm.refcount(1) == 1 and bm.refcount(0) == 8
    _, copy = bm.append_token(0)
    assert copy is None


def pin_free_list_is_a_stack(BM):
    """[P2] "内存分配与回收流程": pop on allocation, push on release; the block released
    last is handed out first; a sequence releases its blocks last first."""
    bm = BM(6, 4, [4, 2, 0, 1, 3, 5])
    bm.add_sequence(0, 8)                       # 4, 2
    bm.add_sequence(1, 4)                       # 0
    assert bm.block_table(0) == [4, 2] and bm.block_table(1) == [0]
    bm.free_sequence(0)                         # pushes 2, then 4
    for sid, want in ((2, 4), (3, 2), (4, 1)):
        bm.add_sequence(sid, 4)
        assert bm.block_table(sid) == [want], (sid, bm.block_table(sid))


def pin_prefix_cache(BM):
    """[P2] "Copy-on-Write 与 Prefix Caching": a prompt whose leading full blocks hold
    the same token prefix as cached blocks references them (counts rise); a different
    first block shares nothing; a partial block is never shared."""
    bm = BM(20, 4)
    a = list(range(1, 11))                      # 2 full blocks + 2 tokens
    assert bm.add_sequence(0, 10, a) == 0
    b = list(range(1, 9)) + [99, 98, 97]
    assert bm.add_sequence(1, 11, b) == 8
    assert bm.block_table(1)[:2] == bm.block_table(0)[:2]
    assert bm.block_table(1)[2] != bm.block_table(0)[2]
    assert bm.refcount(bm.block_table(0)[0]) == 2
    c = [0] + list(range(2, 11))
    assert bm.add_sequence(2, 10, c) == 0
    assert not set(bm.block_table(2)) & set(bm.block_table(0))
    d = [1, 2, 3, 4, 5, 6, 7, 0, 9]
    assert bm.add_sequence(3, 9, d) == 4
    assert bm.block_table(3)[0] == bm.block_table(0)[0]
    assert bm.block_table(3)[1] != bm.block_table(0)[1]
    e = list(range(1, 11))                      # same tokens as a: the partial third block
    assert bm.add_sequence(4, 10, e) == 8       # is not shared
    assert bm.block_table(4)[2] != bm.block_table(0)[2]
    # a block's keys and values depend on every earlier token: a block holding the same
    # 4 tokens behind a different cached first block is not a hit
    assert bm.add_sequence(5, 4, [9, 9, 9, 9]) == 0
    assert bm.add_sequence(6, 8, [9, 9, 9, 9, 5, 6, 7, 8]) == 4
    assert bm.block_table(6)[0] == bm.block_table(5)[0]
    assert bm.block_table(6)[1] != bm.block_table(0)[1]


def pin_lru_eviction(BM):
    """[P2] "BlockAllocator 源码核心": with the free list empty, allocation evicts the
    least recently released cold block; a prefix hit revives a cold block; a request
    that cannot get its blocks fails without changing anything."""
    bm = BM(4, 2)
    bm.add_sequence(0, 4, [1, 2, 3, 4])         # blocks 0, 1, both cached
    bm.free_sequence(0)                         # cold, least recent first: [1, 0]
    assert bm.available() == 4
    bm.add_sequence(1, 2, [7, 8])               # from the free list: 2
    assert bm.block_table(1) == [2]
    assert bm.add_sequence(2, 4, [9, 9, 9, 9]) == 0
    assert bm.block_table(2) == [3, 1]          # free 3, then evicts cold block 1
    try:
        bm.add_sequence(3, 4, [1, 2, 3, 4])     # hits cold block 0, needs 1 more: none
        raise AssertionError("expected NoSpace")
    except NOSPACE:
        pass
    assert bm.available() == 1 and not _exists(bm, 3) and bm.refcount(0) == 0
    bm.free_sequence(1)                         # block 2 goes cold behind 0
    assert bm.add_sequence(3, 4, [1, 2, 3, 4]) == 2
    assert bm.block_table(3) == [0, 2]          # 0 revived, 2 evicted
    assert bm.refcount(0) == 1 and bm.available() == 0


def check_invariants(bm):
    """Every block is exactly one of free / cold / referenced; counts equal the number
    of tables holding the block; the cache maps prefixes to blocks both ways; a live
    sequence's cached full block is cached under that sequence's own token prefix (no
    block is shared between different prefixes); tables hold ceil(n / bs) blocks."""
    n = bm.num_blocks
    free, cold = set(bm.free), set(bm.cold)
    assert len(free) == len(bm.free) and len(cold) == len(bm.cold)
    held = [0] * n
    for t in bm.tables.values():
        for b in t:
            held[b] += 1
    for b in range(n):
        states = (b in free) + (b in cold) + (held[b] > 0)
        assert states == 1, f"block {b}: free {b in free} cold {b in cold} held {held[b]}"
        assert bm.refcount(b) == held[b], f"block {b}: count {bm.refcount(b)} held {held[b]}"
    for key, b in bm.cache.items():
        assert bm.key_of[b] == key
    assert len(bm.cache) == len(bm.key_of)
    assert cold <= set(bm.key_of)
    for sid, t in bm.tables.items():
        nt = bm.num_tokens(sid)
        assert len(t) == (nt + bm.bs - 1) // bm.bs
        toks = bm.tokens[sid]
        if toks is None:
            continue
        for j in range(nt // bm.bs):
            if t[j] in bm.key_of:
                assert bm.key_of[t[j]] == tuple(toks[:(j + 1) * bm.bs]), (sid, j)


def random_ops(BM, seed, steps=400, num_blocks=48, bs=4, check=True, nospace=None):
    """A seeded random serving trace: prompts with shared prefixes, forks, decoded
    tokens, frees; NoSpace is tolerated (and must leave the state whole). Returns the
    list of (operation, result) pairs. `check` runs the oracle's internal invariants
    after every step (oracle class only)."""
    nospace = nospace or NOSPACE
    rng = random.Random(seed)
    bm = BM(num_blocks, bs, rng.sample(range(num_blocks), num_blocks))
    prefixes = [[rng.randrange(50) for _ in range(rng.randrange(0, 13))] for _ in range(4)]
    live, nid, log = [], 0, []
    for _ in range(steps):
        op = rng.random()
        try:
            if op < 0.25 or not live:
                p = rng.choice(prefixes)
                toks = p + [rng.randrange(50) for _ in range(rng.randrange(0, 9))]
                use_ids = rng.random() < 0.8
                got = bm.add_sequence(nid, len(toks), toks if use_ids else None)
                log.append(("add", nid, got, bm.block_table(nid)))
                live.append(nid)
                nid += 1
            elif op < 0.35:
                parent = rng.choice(live)
                bm.fork(parent, nid)
                log.append(("fork", parent, nid, bm.block_table(nid)))
                live.append(nid)
                nid += 1
            elif op < 0.85:
                sid = rng.choice(live)
                got = bm.append_token(sid, rng.randrange(50))
                log.append(("append", sid, got, bm.block_table(sid)))
            else:
                sid = live.pop(rng.randrange(len(live)))
                bm.free_sequence(sid)
                log.append(("free", sid))
        except nospace:
            log.append(("nospace",))
        log.append(("available", bm.available()))
        if check:
            check_invariants(bm)
    return log


def pin_random_invariants(BM):
    for seed in range(6):
        random_ops(BM, seed)


ALL_BM_PINS = [pin_worked_example, pin_allocation_on_demand, pin_copy_on_write,
               pin_free_list_is_a_stack, pin_prefix_cache, pin_lru_eviction,
               pin_random_invariants]
