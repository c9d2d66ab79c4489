"""Host logic of the input generator: block manager and workload shapes (no GPU)."""
import json
import os

import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_block_walk():
    g = _golden("worked_example_fig6.json")
    bs, n = g["block_size"], g["prompt_tokens"]
    order = g["physical_order"] + [x for x in range(12) if x not in g["physical_order"]]
    pool = W.BlockPool(12, order)
    seq = W.prefill(pool, n, bs)
    e = g["expect"]
    assert len(seq.table) == e["logical_blocks_after_prompt"]
    filled = [min(bs, n - j * bs) for j in range(len(seq.table))]
    assert filled == e["filled_per_block"]
    assert len(seq.table) * bs - n == e["free_slots_in_last_block"]
    assert seq.table == e["table_after_prompt"]
    for step in e["decodes"]:
        before = len(seq.table)
        j, off = W.locate(step["position"], bs)
        assert (j, off) == (step["logical_block"], step["offset"])
        slot = W.append_token(pool, seq, bs)
        assert slot == step["slot"]
        assert (len(seq.table) > before) == step["new_block"]
        assert seq.table == step["table_after"]


def test_allocation_on_demand():
    g = _golden("allocation_on_demand.json")
    for c in g["cases"]:
        assert W.blocks_needed(c["tokens"], g["block_size"]) == c["pages"]
    pool = W.BlockPool(4)
    seq = W.prefill(pool, 0, g["block_size"])
    pages = []
    for _ in range(17):
        W.append_token(pool, seq, g["block_size"])
        pages.append(len(seq.table))
    assert pages[4] == 1 and pages[15] == 1 and pages[16] == 2


def test_free_list_refcount_and_release():
    pool = W.BlockPool(5, [4, 2, 0, 1, 3])
    a = W.prefill(pool, 9, 4)
    assert a.table == [4, 2, 0] and pool.num_free() == 2
    b = a.copy_shared(pool)
    assert all(pool.refcount(x) == 2 for x in a.table)
    W.release(pool, a)
    assert pool.num_free() == 2 and all(pool.refcount(x) == 1 for x in b.table)
    W.release(pool, b)
    assert pool.num_free() == 5
    with pytest.raises(W.OutOfBlocks):
        pool.allocate(6)
    with pytest.raises(ValueError):
        pool.decref(4)


def test_copy_on_write_only_forks_written_block():
    pool = W.BlockPool(8)
    a = W.prefill(pool, 6, 4)
    b = a.copy_shared(pool)
    copies = []
    W.append_token(pool, b, 4, copies)
    assert copies == [(a.table[1], b.table[1])]
    assert b.table[0] == a.table[0] and b.table[1] != a.table[1]
    assert pool.refcount(a.table[0]) == 2 and pool.refcount(a.table[1]) == 1
    W.append_token(pool, a, 4, copies)   # the other writer now owns its block alone
    assert len(copies) == 1


def _check_step(s, hq, hkv, d, bs):
    tables, ctx = s.block_tables, s.context_lens
    assert tables.dtype == torch.int32 and ctx.dtype == torch.int32
    assert s.num_heads == hq and s.num_kv_heads == hkv and s.head_dim == d
    used = []
    for b in range(tables.shape[0]):
        nb = W.blocks_needed(int(ctx[b]), bs)
        row = tables[b].tolist()
        assert all(0 <= x < s.num_blocks for x in row[:nb])
        assert all(x == -1 for x in row[nb:])
        used.append(row[:nb])
    return used


def test_llama3_8b_shape():
    s = W.llama3_8b_decode(materialize=False)
    used = _check_step(s, 32, 8, 128, 16)
    ctx = s.context_lens
    assert s.block_tables.shape == (64, 128) and s.num_blocks == 16384
    assert int(ctx.min()) >= 128 and int(ctx.max()) <= 2048
    flat = [x for r in used for x in r]
    assert len(flat) == len(set(flat))          # no sharing in this workload


def test_skewed_shape():
    s = W.skewed_decode(materialize=False)
    used = _check_step(s, 32, 8, 128, 16)
    ctx = s.context_lens.tolist()
    assert s.block_tables.shape == (64, 256) and s.num_blocks == 16384
    assert sorted(ctx)[-1] == 4096 and sorted(ctx)[-2] <= 512 and min(ctx) >= 128
    flat = [x for r in used for x in r]
    assert len(flat) == len(set(flat))


def test_llama_70b_shape():
    s = W.llama_70b_decode(materialize=False)
    used = _check_step(s, 64, 8, 128, 16)
    ctx = s.context_lens.double()
    assert int(ctx.min()) >= 16 and int(ctx.max()) <= 4096
    assert 700 < float(ctx.median()) < 1400
    need = sum(len(r) for r in used)
    assert s.num_blocks == -(-11 * need // 10)


def test_long_context_shape():
    s = W.long_context_decode(materialize=False)
    _check_step(s, 32, 8, 128, 16)
    assert int(s.context_lens.min()) >= 32768 and int(s.context_lens.max()) <= 131072
    assert s.partition_size == 512


@pytest.mark.parametrize("prefix", [2048, 2040])
def test_shared_prefix_structure(prefix):
    s = W.shared_prefix_cow(materialize=False, prefix_tokens=prefix)
    used = _check_step(s, 32, 8, 128, 16)
    nbp = W.blocks_needed(prefix, 16)
    pairs = s.copy_pairs.tolist()
    assert len(pairs) == 32 * 7
    dsts = [p[1] for p in pairs]
    srcs = {p[0] for p in pairs}
    assert len(set(dsts)) == len(dsts) and not (set(dsts) & srcs)
    for p in range(32):
        group = used[p * 8:(p + 1) * 8]
        for s_ in group[1:]:                       # full prefix blocks shared ...
            assert s_[:nbp - 1] == group[0][:nbp - 1]
        lasts = {g[nbp - 1] for g in group}        # ... the last prefix block forked
        assert len(lasts) == 8
    slots = s.slot_mapping.tolist()
    assert len(slots) == len(set(slots))
    div = s.extra["divergent"]
    assert s.context_lens.tolist() == [prefix + d + 1 for d in div]
    assert len(slots) == sum(d + 1 for d in div)


def test_tiny_fp32_recipe():
    s = W.tiny_fp32()
    assert s.context_lens_before.tolist() == [7, 16, 33, 100]
    assert s.context_lens.tolist() == [8, 17, 34, 101]
    assert s.block_tables.shape == (4, 26)
    # appends at positions 7, 16, 33, 100 land at (block, offset) (1,3) (4,0) (8,1) (25,0)
    for b, (j, off) in enumerate([(1, 3), (4, 0), (8, 1), (25, 0)]):
        slot = int(s.slot_mapping[b])
        assert slot == int(s.block_tables[b, j]) * 4 + off
    pairs = s.copy_pairs.tolist()
    used = {x for x in s.block_tables.flatten().tolist() if x >= 0}
    assert len(pairs) == 3 and all(a in used and b not in used for a, b in pairs)
    assert s.q.shape == (4, 8, 64) and s.k_cache.shape == (64, 8, 4, 64)


def test_generators_are_deterministic():
    a, b = W.tiny_fp32(), W.tiny_fp32()
    assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.block_tables, b.block_tables)
    c, d = W.llama3_8b_decode(materialize=False), W.llama3_8b_decode(materialize=False)
    assert torch.equal(c.block_tables, d.block_tables)
