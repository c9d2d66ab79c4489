"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Every ``pin_*`` function takes a loaded oracle library (``lib``) and raises
AssertionError when the oracle disagrees with:
  * the pages' worked example (tests/golden/*.json, each with its citation),
  * a closed form derived by hand or from the definition (ctx = 1, uniform
    scores, a two-token case),
  * a library routine on the un-paged data (torch's scaled_dot_product_attention
    in float64 on the contiguous sequence, torch's dtype conversions),
  * an invariant of the method (placement permutation, grouped-query = repeated
    multi-head, stale slots never read, linearity in V, write-then-read identity
    of the append, copy-on-write isolation),
  * the NumPy dense brute force, a second, independently written definition.
The same functions run against deliberately broken builds of the oracle in
tests/test_oracle_mutants.py: each planted mistake must trip at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from workloads import BlockPool, append_token, blocks_needed, pack_tables, prefill, slot_of

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- helpers
def paged_from_contiguous(keys, values, bs, num_blocks, order, dtype, fill=0.0, seed=0):
    """Scatter per-sequence contiguous K/V ([n_b, Hkv, D] each) into a paged pool.

    Placement uses the block manager (free-list order ``order``); every slot not
    holding a token gets ``fill`` (NaN poisons stale slots, padding and free blocks)
    or, with fill=None, random values. Returns (k_cache, v_cache, tables, ctx).
    """
    hkv, d = keys[0].shape[1], keys[0].shape[2]
    pool = BlockPool(num_blocks, order)
    seqs = [prefill(pool, k.shape[0], bs) for k in keys]
    if fill is None:
        g = torch.Generator().manual_seed(seed)
        kc = torch.randn(num_blocks, hkv, bs, d, generator=g, dtype=torch.float64)
        vc = torch.randn(num_blocks, hkv, bs, d, generator=g, dtype=torch.float64)
    else:
        kc = torch.full((num_blocks, hkv, bs, d), float(fill), dtype=torch.float64)
        vc = torch.full((num_blocks, hkv, bs, d), float(fill), dtype=torch.float64)
    for s, k, v in zip(seqs, keys, values):
        for t in range(k.shape[0]):
            slot = slot_of(s, t, bs)
            kc[slot // bs, :, slot % bs, :] = k[t].to(torch.float64)
            vc[slot // bs, :, slot % bs, :] = v[t].to(torch.float64)
    width = max(1, max(len(s.table) for s in seqs))
    tables = torch.tensor(pack_tables(seqs, width), dtype=torch.int32)
    ctx = torch.tensor([k.shape[0] for k in keys], dtype=torch.int32)
    return kc.to(dtype), vc.to(dtype), tables, ctx


def sdpa_reference(q, keys, values, scale):
    """Library attention on the contiguous (un-paged) sequences, float64.

    q [B, Hq, D]; keys[b], values[b] [n_b, Hkv, D]. Grouped heads are expanded by
    repeat_interleave (query head h reads KV head h // group)."""
    B, Hq, D = q.shape
    out = torch.zeros(B, Hq, D, dtype=torch.float64)
    for b in range(B):
        n = keys[b].shape[0]
        if n == 0:
            continue
        hkv = keys[b].shape[1]
        K = keys[b].to(torch.float64).permute(1, 0, 2).repeat_interleave(Hq // hkv, dim=0)
        V = values[b].to(torch.float64).permute(1, 0, 2).repeat_interleave(Hq // hkv, dim=0)
        qq = q[b].to(torch.float64).unsqueeze(1)           # [Hq, 1, D]
        out[b] = F.scaled_dot_product_attention(qq, K, V, scale=float(scale)).squeeze(1)
    return out.numpy()


def _random_seqs(seed, lens, hkv, d, dtype):
    g = torch.Generator().manual_seed(seed)
    keys = [torch.randn(n, hkv, d, generator=g).to(dtype) for n in lens]
    values = [torch.randn(n, hkv, d, generator=g).to(dtype) for n in lens]
    return keys, values


def _order(seed, n):
    return torch.randperm(n, generator=torch.Generator().manual_seed(seed)).tolist()


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


DTYPES = (torch.float32, torch.bfloat16, torch.float16)


# ----------------------------------------------------------------------------- pins
def pin_decoders(lib):
    """Every bf16 and f16 bit pattern decodes to what torch's conversion gives."""
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    for dt in (torch.bfloat16, torch.float16):
        t = bits.view(dt)
        got = oracle.decode(t, lib=lib)
        want = t.to(torch.float64).numpy()
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), f"{dt}: NaN set differs"
        assert np.array_equal(got[~nan], want[~nan]), f"{dt}: decoded values differ"
    x = torch.randn(1000, generator=torch.Generator().manual_seed(5))
    assert np.array_equal(oracle.decode(x, lib=lib), x.double().numpy())


def pin_sdpa_library(lib):
    """Paged walk == library attention on the contiguous sequences (all dtypes,
    several block sizes, grouped heads, ragged lengths incl. 1 and block multiples)."""
    cases = [(1, 4, 4, 8, [5, 1, 12, 9]), (4, 8, 2, 64, [7, 16, 33, 40]),
             (16, 4, 1, 16, [31, 16, 17]), (2, 8, 8, 32, [3, 4, 1, 6])]
    for i, (bs, hq, hkv, d, lens) in enumerate(cases):
        for dt in DTYPES:
            keys, values = _random_seqs(100 + i, lens, hkv, d, dt)
            need = sum(blocks_needed(n, bs) for n in lens) + 5
            kc, vc, tables, ctx = paged_from_contiguous(keys, values, bs, need, _order(i, need),
                                                        dt, fill=None, seed=i)
            q = torch.randn(len(lens), hq, d, generator=torch.Generator().manual_seed(i)).to(dt)
            scale = 1.0 / math.sqrt(d)
            got = oracle.paged_attention(q, kc, vc, tables, ctx, scale, lib=lib)
            _close(got, sdpa_reference(q, keys, values, scale), 1e-12, f"sdpa case {i} {dt}")


def pin_dense_bruteforce(lib):
    """C walk == NumPy dense gather-then-softmax on random tiny batches."""
    from workloads import random_small
    shapes = [(3, 2, 2, 8, 1, 9), (4, 8, 2, 64, 4, 40), (2, 8, 1, 8, 16, 40), (4, 4, 4, 16, 2, 23)]
    for i, (B, hq, hkv, d, bs, mx) in enumerate(shapes):
        for dt in DTYPES:
            s = random_small(200 + i, batch=B, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                             block_size=bs, max_ctx=mx, dtype=dt)
            got = oracle.paged_attention(s.q, s.k_cache, s.v_cache, s.block_tables,
                                         s.context_lens, s.scale, lib=lib)
            want = oracle.dense_attention(s.q, s.k_cache, s.v_cache, s.block_tables,
                                          s.context_lens, s.scale)
            scale = max(1.0, float(np.max(np.abs(want))))
            _close(got / scale, want / scale, 1e-12, f"dense case {i} {dt}")


def pin_dense_vs_library():
    """The NumPy brute force itself matches the library attention (pins dense.py)."""
    lens = [9, 1, 20]
    keys, values = _random_seqs(7, lens, 2, 16, torch.float32)
    kc, vc, tables, ctx = paged_from_contiguous(keys, values, 4, 20, _order(3, 20),
                                                torch.float32, fill=None, seed=1)
    q = torch.randn(3, 4, 16, generator=torch.Generator().manual_seed(2))
    got = oracle.dense_attention(q, kc, vc, tables, ctx, 0.25)
    _close(got, sdpa_reference(q, keys, values, 0.25), 1e-12, "dense vs sdpa")


def pin_worked_example(lib):
    """The pages' block-size-4 walk-through: a 7-token prompt placed on physical
    blocks 5 and 3, the 8th token fills the free slot, the 9th opens block 8; after
    each append the decode equals attention over the contiguous 8 and 9 tokens."""
    g = _golden("worked_example_fig6.json")
    bs, n0 = g["block_size"], g["prompt_tokens"]
    order = list(g["physical_order"]) + [x for x in range(10) if x not in g["physical_order"]]
    hkv, hq, d = 2, 4, 8
    gen = torch.Generator().manual_seed(11)
    K = torch.randn(n0 + 2, hkv, d, generator=gen, dtype=torch.float64)
    V = torch.randn(n0 + 2, hkv, d, generator=gen, dtype=torch.float64)
    q = torch.randn(1, hq, d, generator=gen, dtype=torch.float64).to(torch.float32)
    K, V = K.to(torch.float32), V.to(torch.float32)
    kc, vc, tables, ctx = paged_from_contiguous([K[:n0]], [V[:n0]], bs, 10, order,
                                                torch.float32, fill=float("nan"))
    assert tables[0, :2].tolist() == g["expect"]["table_after_prompt"]
    pool = BlockPool(10, order)
    seq = prefill(pool, n0, bs)
    for step in g["expect"]["decodes"]:
        slot = append_token(pool, seq, bs)
        assert slot == step["slot"], f"slot {slot} != {step['slot']}"
        assert seq.table == step["table_after"]
        pos = step["position"]
        # the decode step's own slot rule: the walk to position ctx - 1
        tb_now = torch.tensor([seq.table], dtype=torch.int32)
        got_slot = oracle.context_end_slots(tb_now, torch.tensor([pos + 1]), bs)
        assert got_slot.tolist() == [step["slot"]], f"context-end slot {got_slot.tolist()}"
        assert step["logical_block"] == pos // bs and step["offset"] == pos % bs
        kc, vc = oracle.reshape_and_cache(K[pos:pos + 1], V[pos:pos + 1], kc, vc,
                                          torch.tensor([slot]), lib=lib)
        tb = torch.tensor([seq.table + [-1] * (3 - len(seq.table))], dtype=torch.int32)
        got = oracle.paged_attention(q, kc, vc, tb, torch.tensor([pos + 1], dtype=torch.int32),
                                     0.3, lib=lib)
        want = sdpa_reference(q, [K[:pos + 1]], [V[:pos + 1]], 0.3)
        _close(got, want, 1e-12, f"worked example after token {step['token_number']}")


def pin_two_token_closed_form(lib):
    g = _golden("two_token_closed_form.json")
    keys = torch.tensor(g["keys"], dtype=torch.float32).unsqueeze(1)     # [2, 1, 2]
    values = torch.tensor(g["values"], dtype=torch.float32).unsqueeze(1)
    kc, vc, tables, ctx = paged_from_contiguous([keys], [values], g["block_size"], 2,
                                                g["physical_order"], torch.float32,
                                                fill=float("nan"))
    q = torch.tensor([[g["q"]]], dtype=torch.float32)
    got = oracle.paged_attention(q, kc, vc, tables, ctx, g["scale"], lib=lib)
    _close(got.reshape(-1), g["expect"], g["tolerance"], "two-token closed form")


def pin_context_one(lib):
    """A single token gets weight exactly one: the output is v0, bit for bit."""
    for dt in DTYPES:
        keys, values = _random_seqs(31, [1, 1], 2, 16, dt)
        kc, vc, tables, ctx = paged_from_contiguous(keys, values, 4, 6, _order(1, 6), dt,
                                                    fill=None, seed=4)
        q = torch.randn(2, 4, 16, generator=torch.Generator().manual_seed(3)).to(dt)
        got = oracle.paged_attention(q, kc, vc, tables, ctx, 0.25, lib=lib)
        want = torch.stack([v[0].repeat_interleave(2, dim=0) for v in values]).double().numpy()
        assert np.array_equal(got, want), f"ctx=1 {dt}"


def pin_uniform_scores(lib):
    """q = 0 (or scale = 0) makes every score equal: the output is the mean of V."""
    lens = [13, 4, 32]
    keys, values = _random_seqs(41, lens, 2, 8, torch.float32)
    kc, vc, tables, ctx = paged_from_contiguous(keys, values, 4, 20, _order(2, 20),
                                                torch.float32, fill=None, seed=6)
    want = np.stack([v.double().mean(0).repeat_interleave(2, dim=0).numpy() for v in values])
    q0 = torch.zeros(3, 4, 8)
    _close(oracle.paged_attention(q0, kc, vc, tables, ctx, 0.5, lib=lib), want, 1e-12, "q=0")
    q1 = torch.randn(3, 4, 8, generator=torch.Generator().manual_seed(8))
    _close(oracle.paged_attention(q1, kc, vc, tables, ctx, 0.0, lib=lib), want, 1e-12,
           "scale=0")


def pin_zero_context(lib):
    """Reading taken: an empty context gives a zero output (and other rows unaffected)."""
    keys, values = _random_seqs(51, [0, 5], 1, 8, torch.float32)
    kc, vc, tables, ctx = paged_from_contiguous(keys, values, 4, 4, _order(5, 4),
                                                torch.float32, fill=None, seed=2)
    q = torch.randn(2, 1, 8, generator=torch.Generator().manual_seed(9))
    got = oracle.paged_attention(q, kc, vc, tables, ctx, 0.3, lib=lib)
    assert np.array_equal(got[0], np.zeros((1, 8)))
    _close(got[1:], sdpa_reference(q[1:], keys[1:], values[1:], 0.3), 1e-12, "row after empty")


def pin_placement_permutation(lib):
    """The same tokens on a different physical placement give the identical output."""
    lens = [7, 16, 33, 21]
    for dt in (torch.float32, torch.bfloat16):
        keys, values = _random_seqs(61, lens, 2, 16, dt)
        q = torch.randn(4, 8, 16, generator=torch.Generator().manual_seed(12)).to(dt)
        outs = []
        for perm_seed in (1, 2, 3):
            kc, vc, tables, ctx = paged_from_contiguous(keys, values, 4, 30,
                                                        _order(perm_seed, 30), dt, fill=None,
                                                        seed=perm_seed)
            outs.append(oracle.paged_attention(q, kc, vc, tables, ctx, 0.25, lib=lib))
        assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2]), dt


def pin_gqa_equals_repeated_mha(lib):
    """Grouped-query attention equals multi-head attention with each KV head repeated
    for its group (query head h reads KV head h // group)."""
    lens = [9, 20, 4]
    hkv, group, d = 2, 4, 16
    keys, values = _random_seqs(71, lens, hkv, d, torch.float32)
    q = torch.randn(3, hkv * group, d, generator=torch.Generator().manual_seed(13))
    kc, vc, tables, ctx = paged_from_contiguous(keys, values, 4, 12, _order(4, 12),
                                                torch.float32, fill=None, seed=3)
    got = oracle.paged_attention(q, kc, vc, tables, ctx, 0.25, lib=lib)
    rk = [k.repeat_interleave(group, dim=1) for k in keys]
    rv = [v.repeat_interleave(group, dim=1) for v in values]
    kc2, vc2, tables2, ctx2 = paged_from_contiguous(rk, rv, 4, 12, _order(4, 12),
                                                    torch.float32, fill=None, seed=3)
    want = oracle.paged_attention(q, kc2, vc2, tables2, ctx2, 0.25, lib=lib)
    assert np.array_equal(got, want)


def pin_stale_slots_unread(lib):
    """NaN in the unfilled slots of last blocks, in table padding targets and in free
    blocks changes nothing (only tokens below the context length are read)."""
    lens = [7, 16, 2]
    keys, values = _random_seqs(81, lens, 2, 8, torch.float32)
    q = torch.randn(3, 4, 8, generator=torch.Generator().manual_seed(14))
    a = paged_from_contiguous(keys, values, 4, 12, _order(6, 12), torch.float32, fill=0.0)
    b = paged_from_contiguous(keys, values, 4, 12, _order(6, 12), torch.float32,
                              fill=float("nan"))
    ra = oracle.paged_attention(q, a[0], a[1], a[2], a[3], 0.3, lib=lib)
    rb = oracle.paged_attention(q, b[0], b[1], b[2], b[3], 0.3, lib=lib)
    assert np.all(np.isfinite(rb)) and np.array_equal(ra, rb)


def pin_linearity_in_values(lib):
    """The output is linear in V for fixed q and K."""
    lens = [11, 5]
    keys, v1 = _random_seqs(91, lens, 1, 8, torch.float64)
    _, v2 = _random_seqs(92, lens, 1, 8, torch.float64)
    q = torch.randn(2, 2, 8, generator=torch.Generator().manual_seed(15))
    outs = []
    for vals in (v1, v2, [a + 2.0 * b for a, b in zip(v1, v2)]):
        kc, vc, tables, ctx = paged_from_contiguous(keys, vals, 4, 8, _order(7, 8),
                                                    torch.float32, fill=None, seed=5)
        outs.append(oracle.paged_attention(q, kc, vc, tables, ctx, 0.3, lib=lib))
    # values were rounded to float32 when placed; compare in that precision
    _close(outs[2], outs[0] + 2.0 * outs[1], 1e-5, "linearity")


def pin_append_roundtrip(lib):
    """Writing a sequence token by token through the slot mapping and reading it back
    through the block table returns the sequence; nothing else in the pool changes;
    negative slots write nothing."""
    for dt in DTYPES:
        bs, hkv, d, nb = 4, 3, 8, 16
        gen = torch.Generator().manual_seed(17)
        kc0 = torch.randn(nb, hkv, bs, d, generator=gen).to(dt)
        vc0 = torch.randn(nb, hkv, bs, d, generator=gen).to(dt)
        pool = BlockPool(nb, _order(8, nb))
        seqs = [prefill(pool, 0, bs) for _ in range(3)]
        lens = [6, 9, 4]
        slots, toks = [], []
        for step in range(max(lens)):
            for i, s in enumerate(seqs):
                if step < lens[i]:
                    slots.append(append_token(pool, s, bs))
                    toks.append((i, step))
                    slots.append(-1)            # padding entry: must write nothing
                    toks.append(None)
        T = len(slots)
        newk = torch.randn(T, hkv, d, generator=gen).to(dt)
        newv = torch.randn(T, hkv, d, generator=gen).to(dt)
        kc, vc = oracle.reshape_and_cache(newk, newv, kc0, vc0,
                                          torch.tensor(slots, dtype=torch.int64), lib=lib)
        written = torch.zeros(nb, bs, dtype=torch.bool)
        for t, tok in enumerate(toks):
            if tok is None:
                continue
            i, pos = tok
            blk = seqs[i].table[pos // bs]
            assert torch.equal(kc[blk, :, pos % bs], newk[t]), "K not readable at its position"
            assert torch.equal(vc[blk, :, pos % bs], newv[t]), "V not readable at its position"
            written[blk, pos % bs] = True
        keep = ~written
        assert torch.equal(kc.permute(0, 2, 1, 3)[keep], kc0.permute(0, 2, 1, 3)[keep])
        assert torch.equal(vc.permute(0, 2, 1, 3)[keep], vc0.permute(0, 2, 1, 3)[keep])


def pin_copy_on_write(lib):
    """Copy-on-write through the block manager: two sequences share a partly filled
    block; before the second one writes, the block is copied. Afterwards the first
    sequence still sees its old tokens, the writer sees the shared prefix plus its
    new token, and every other block is untouched."""
    for dt in (torch.float32, torch.bfloat16):
        bs, hkv, d, nb = 4, 2, 8, 10
        gen = torch.Generator().manual_seed(19)
        kc0 = torch.randn(nb, hkv, bs, d, generator=gen).to(dt)
        pool = BlockPool(nb, _order(9, nb))
        a = prefill(pool, 6, bs)
        b = a.copy_shared(pool)
        copies = []
        slot = append_token(pool, b, bs, copies)
        assert len(copies) == 1 and copies[0][0] == a.table[1] and b.table[1] == copies[0][1]
        assert b.table[0] == a.table[0] and pool.refcount(a.table[0]) == 2
        kc = oracle.copy_blocks(kc0, torch.tensor(copies, dtype=torch.int32), lib=lib)
        src, dst = copies[0]
        assert torch.equal(kc[dst], kc0[src]), "copy does not hold the source block"
        others = [x for x in range(nb) if x != dst]
        assert torch.equal(kc[others], kc0[others]), "copy touched another block"
        newk = torch.randn(1, hkv, d, generator=gen).to(dt)
        kc2, _ = oracle.reshape_and_cache(newk, newk, kc, kc.clone(),
                                          torch.tensor([slot]), lib=lib)
        for pos in range(6):   # the first sequence's view is unchanged
            blk = a.table[pos // bs]
            assert torch.equal(kc2[blk, :, pos % bs], kc0[blk, :, pos % bs])
        for pos in range(6):   # the writer sees the same prefix ...
            blk = b.table[pos // bs]
            assert torch.equal(kc2[blk, :, pos % bs], kc0[a.table[pos // bs], :, pos % bs])
        assert torch.equal(kc2[b.table[1], :, 6 % bs], newk[0])   # ... and its new token


def pin_decode_step_slots(lib):
    """The decode step appends at the context end. For sequences grown token by token
    through the block manager, whose allocation path is independent of the oracle,
    the context-end slot of every sequence is the slot its last append returned.
    Empty contexts write nothing. The composed step equals an explicit append
    followed by attention over the contiguous tokens."""
    bs, nb = 4, 24
    pool = BlockPool(nb, _order(21, nb))
    lens = [5, 8, 1, 0, 12, 9]
    seqs, last = [], []
    for n in lens:
        s = prefill(pool, max(n - 1, 0), bs)
        last.append(append_token(pool, s, bs) if n > 0 else -1)
        seqs.append(s)
    tables = torch.tensor(pack_tables(seqs, 4), dtype=torch.int32)
    ctx = torch.tensor(lens, dtype=torch.int32)
    assert oracle.context_end_slots(tables, ctx, bs).tolist() == last
    hkv, hq, d = 2, 4, 8
    gen = torch.Generator().manual_seed(23)
    K = [torch.randn(n, hkv, d, generator=gen) for n in lens]
    V = [torch.randn(n, hkv, d, generator=gen) for n in lens]
    kc = torch.full((nb, hkv, bs, d), float("nan"))
    vc = torch.full((nb, hkv, bs, d), float("nan"))
    for i, s in enumerate(seqs):           # every token but the newest is already cached
        for t in range(lens[i] - 1):
            kc[s.table[t // bs], :, t % bs] = K[i][t]
            vc[s.table[t // bs], :, t % bs] = V[i][t]
    newk = torch.stack([K[i][-1] if lens[i] else torch.zeros(hkv, d) for i in range(len(lens))])
    newv = torch.stack([V[i][-1] if lens[i] else torch.zeros(hkv, d) for i in range(len(lens))])
    q = torch.randn(len(lens), hq, d, generator=gen)
    out, ek, ev = oracle.decode_step(q, newk, newv, kc, vc, tables, ctx, 0.35, lib=lib)
    want = sdpa_reference(q, K, V, 0.35)
    _close(out, want, 1e-12, "decode step vs contiguous attention")
    assert np.all(out[3] == 0), "empty context"
    for i, s in enumerate(seqs):
        if lens[i]:
            p = lens[i] - 1
            assert torch.equal(ek[s.table[p // bs], :, p % bs], K[i][-1])
            assert torch.equal(ev[s.table[p // bs], :, p % bs], V[i][-1])


# ------------------------------------------------------------------ 8-bit KV cache
def _fp8_values(codes):
    """Values of E4M3 codes through torch's float8_e4m3fn type (a library routine)."""
    return codes.view(torch.float8_e4m3fn).to(torch.float64)


def _random_codes(shape, gen):
    """Random finite E4M3 codes (both signs, NaN codes excluded)."""
    mag = torch.randint(0, 0x7F, shape, generator=gen, dtype=torch.int32)
    sign = torch.randint(0, 2, shape, generator=gen, dtype=torch.int32) * 0x80
    return (mag | sign).to(torch.uint8)


def pin_fp8_decode(lib):
    """Every OCP E4M3 code decodes to the value torch's float8_e4m3fn type gives it
    (NaN codes included); closed forms: 448 is the largest finite value, 2^-9 the
    smallest subnormal, 0x38 is one."""
    codes = torch.arange(256, dtype=torch.uint8)
    got = oracle.fp8_decode(codes, lib=lib)
    want = _fp8_values(codes).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want)), "NaN codes"
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin]), "decoded values"
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0


def pin_fp8_quantize(lib):
    """Quantisation to E4M3: every finite code round-trips; a value midway between
    neighbouring codes goes to the one with the even mantissa; random in-range values
    (normal and subnormal) match torch's conversion; 448 and beyond (infinity too)
    saturate to 448, NaN stays NaN; the scale enters as one binary32 product."""
    codes = torch.arange(256, dtype=torch.uint8)
    vals = _fp8_values(codes).to(torch.float32)
    fin = ~torch.isnan(vals)
    assert torch.equal(oracle.fp8_quantize(vals[fin], 1.0, lib=lib), codes[fin]), "round trip"
    for sign in (1.0, -1.0):
        pos = vals[:0x7F].double() * sign
        mids = ((pos[:-1] + pos[1:]) / 2).to(torch.float32)   # exact in float32
        lo = torch.arange(0, 0x7E, dtype=torch.int32)
        even = torch.where(lo % 2 == 0, lo, lo + 1) | (0x80 if sign < 0 else 0)
        got = oracle.fp8_quantize(mids, 1.0, lib=lib).to(torch.int32)
        assert torch.equal(got, even), f"ties to even ({sign:+.0f})"
    g = torch.Generator().manual_seed(31)
    for x in ((torch.rand(20000, generator=g) * 2 - 1) * 447.0,
              torch.randn(20000, generator=g) * 0.02,            # subnormal range too
              torch.randn(20000, generator=g) * 3.0):
        want = x.to(torch.float8_e4m3fn).view(torch.uint8)
        assert torch.equal(oracle.fp8_quantize(x, 1.0, lib=lib), want), "vs torch"
    # [464, 480) would round up to the NaN code without saturation
    sat = torch.tensor([448.0, 449.0, 463.9, 464.0, 470.0, 479.99, 1e6, float("inf"),
                        -448.0, -470.0, -1e6, -float("inf")])
    assert oracle.fp8_quantize(sat, 1.0, lib=lib).tolist() == [0x7E] * 8 + [0xFE] * 4
    nan = oracle.fp8_quantize(torch.tensor([float("nan")]), 1.0, lib=lib)
    assert int(nan[0]) & 0x7F == 0x7F, "NaN"
    xb = torch.randn(5000, generator=g).to(torch.bfloat16)
    inv = oracle.inv_scale(0.0123)
    prod = xb.to(torch.float32) * torch.tensor(inv, dtype=torch.float32)
    assert torch.equal(oracle.fp8_quantize(xb, inv, lib=lib),
                       oracle.fp8_quantize(prod, 1.0, lib=lib)), "binary32 product"


def pin_fp8_attention(lib):
    """Attention over 8-bit caches equals the plain definition on the dequantised
    values (torch's float8 decode times the scales, then the NumPy brute force)."""
    bs, hkv, hq, d, nb = 4, 2, 4, 16, 24
    g = torch.Generator().manual_seed(37)
    kc = _random_codes((nb, hkv, bs, d), g)
    vc = _random_codes((nb, hkv, bs, d), g)
    ks, vs = 0.0173, 0.25
    pool = BlockPool(nb, _order(39, nb))
    lens = [7, 1, 0, 16, 21]
    seqs = [prefill(pool, n, bs) for n in lens]
    tables = torch.tensor(pack_tables(seqs, 6), dtype=torch.int32)
    ctx = torch.tensor(lens, dtype=torch.int32)
    q = torch.randn(len(lens), hq, d, generator=g).to(torch.bfloat16)
    got = oracle.paged_attention_fp8(q, kc, vc, ks, vs, tables, ctx, 0.3, lib=lib)
    want = oracle.dense_attention(q, _fp8_values(kc) * ks, _fp8_values(vc) * vs, tables, ctx,
                                  0.3)
    _close(got, want, 1e-12, "fp8 attention vs dequantised brute force")


def pin_fp8_append(lib):
    """The quantising append writes, at each token's slot, torch's E4M3 conversion of
    float32(x) * float32(1/scale) (K and V with their own scales), and changes nothing
    else; negative slots write nothing."""
    bs, hkv, d, nb = 4, 3, 8, 12
    g = torch.Generator().manual_seed(41)
    kc0, vc0 = _random_codes((nb, hkv, bs, d), g), _random_codes((nb, hkv, bs, d), g)
    pool = BlockPool(nb, _order(43, nb))
    seq = prefill(pool, 0, bs)
    slots = [append_token(pool, seq, bs) for _ in range(6)] + [-1]
    T = len(slots)
    newk = torch.randn(T, hkv, d, generator=g).to(torch.bfloat16)
    newv = (torch.randn(T, hkv, d, generator=g) * 5).to(torch.bfloat16)
    ks, vs = 0.011, 0.07
    kc, vc = oracle.reshape_and_cache_fp8(newk, newv, kc0, vc0,
                                          torch.tensor(slots, dtype=torch.int64), ks, vs,
                                          lib=lib)

    def conv(x, scale):
        inv = torch.tensor(oracle.inv_scale(scale), dtype=torch.float32)
        return (x.to(torch.float32) * inv).to(torch.float8_e4m3fn).view(torch.uint8)

    touched = torch.zeros(nb, bs, dtype=torch.bool)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = slot // bs, slot % bs
        assert torch.equal(kc[blk, :, off], conv(newk[t], ks)), "K codes"
        assert torch.equal(vc[blk, :, off], conv(newv[t], vs)), "V codes"
        touched[blk, off] = True
    keep = ~touched
    assert torch.equal(kc.permute(0, 2, 1, 3)[keep], kc0.permute(0, 2, 1, 3)[keep])
    assert torch.equal(vc.permute(0, 2, 1, 3)[keep], vc0.permute(0, 2, 1, 3)[keep])


# ----------------------------------------------------------------------------- chunks
def _chunk_case(seed, lens, tlens, hq, hkv, d, bs, dt):
    """Contiguous sequences of lengths `lens` placed in a paged pool (random filler
    elsewhere), plus tlens[b] query rows per sequence. Returns the pieces for both the
    paged oracle and library references."""
    keys, values = _random_seqs(seed, lens, hkv, d, dt)
    need = sum(blocks_needed(n, bs) for n in lens) + 4
    kc, vc, tables, ctx = paged_from_contiguous(keys, values, bs, need, _order(seed, need), dt,
                                                fill=None, seed=seed)
    qs = torch.tensor([0] + list(np.cumsum(tlens)), dtype=torch.int32)
    g = torch.Generator().manual_seed(seed + 1)
    q = torch.randn(int(qs[-1]), hq, d, generator=g).to(dt)
    return keys, values, kc, vc, tables, ctx, qs, q


def pin_chunk_causal_sdpa(lib):
    """Several query tokens per sequence == library attention with an explicit causal
    mask on the contiguous sequence: row j of a T-token chunk (position n - T + j) keeps
    the tokens at positions <= n - T + j. Covers single-token chunks, whole prompts
    (T = n), empty chunks, block sizes 1/4/16 and grouped heads."""
    cases = [(4, 8, 2, 16, [9, 16, 33, 5], [3, 1, 33, 0]),
             (16, 4, 4, 32, [40, 17], [16, 5]),
             (1, 6, 3, 8, [6, 2, 11], [6, 2, 4])]
    for i, (bs, hq, hkv, d, lens, tl) in enumerate(cases):
        for dt in DTYPES:
            keys, values, kc, vc, tables, ctx, qs, q = _chunk_case(300 + i, lens, tl, hq, hkv,
                                                                   d, bs, dt)
            scale = 1.0 / math.sqrt(d)
            got = oracle.paged_attention_chunk(q, kc, vc, tables, ctx, qs, scale, lib=lib)
            want = np.zeros_like(got)
            for b, (n, T) in enumerate(zip(lens, tl)):
                if T == 0:
                    continue
                r0 = int(qs[b])
                K = keys[b].to(torch.float64).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
                V = values[b].to(torch.float64).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
                Q = q[r0:r0 + T].to(torch.float64).permute(1, 0, 2)          # [Hq, T, D]
                keep = torch.arange(n)[None, :] <= (n - T + torch.arange(T))[:, None]
                o = F.scaled_dot_product_attention(Q, K, V, attn_mask=keep, scale=scale)
                want[r0:r0 + T] = o.permute(1, 0, 2).numpy()
            _close(got, want, 1e-12, f"chunk sdpa case {i} {dt}")


def pin_chunk_dense(lib):
    """Chunk walk == the NumPy masked dense form on random batches, including rows
    whose position falls before the context (more query rows than tokens): zero."""
    from workloads import random_small
    g = torch.Generator().manual_seed(77)
    for i, (B, hq, hkv, d, bs, mx) in enumerate([(4, 8, 2, 16, 4, 40), (3, 4, 4, 8, 16, 50),
                                                 (5, 2, 1, 8, 2, 9)]):
        for dt in DTYPES:
            s = random_small(400 + i, batch=B, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                             block_size=bs, max_ctx=mx, dtype=dt)
            ctx = s.context_lens.tolist()
            tl = [int(torch.randint(0, n + 1, (1,), generator=g)) for n in ctx]
            tl[0] = ctx[0] + 2                       # two rows before the context starts
            qs = torch.tensor([0] + list(np.cumsum(tl)), dtype=torch.int32)
            q = torch.randn(int(qs[-1]), hq, d, generator=g).to(dt)
            got = oracle.paged_attention_chunk(q, s.k_cache, s.v_cache, s.block_tables,
                                               s.context_lens, qs, s.scale, lib=lib)
            want = oracle.dense_chunk_attention(q, s.k_cache, s.v_cache, s.block_tables,
                                                s.context_lens, qs, s.scale)
            assert np.all(got[:2] == 0.0), "rows before the context must be zero"
            _close(got, want, 1e-12, f"chunk dense case {i} {dt}")


def pin_chunk_causality(lib):
    """Changing the key and value of the token at position p leaves every query row at
    a position < p bit for bit unchanged, and changes the rows at positions >= p."""
    bs, hq, hkv, d = 4, 4, 2, 8
    lens, tl = [13, 9], [6, 9]
    keys, values, kc, vc, tables, ctx, qs, q = _chunk_case(500, lens, tl, hq, hkv, d, bs,
                                                           torch.float32)
    base = oracle.paged_attention_chunk(q, kc, vc, tables, ctx, qs, 0.4, lib=lib)
    for b, p in ((0, 10), (1, 4)):
        kc2, vc2 = kc.clone(), vc.clone()
        blk = int(tables[b, p // bs])
        kc2[blk, :, p % bs] += 3.0
        vc2[blk, :, p % bs] -= 2.0
        got = oracle.paged_attention_chunk(q, kc2, vc2, tables, ctx, qs, 0.4, lib=lib)
        r0, n, T = int(qs[b]), lens[b], tl[b]
        for j in range(T):
            pos = n - T + j
            same = np.array_equal(got[r0 + j], base[r0 + j])
            assert same == (pos < p), f"seq {b} row {j} (position {pos}) vs change at {p}"


def pin_chunk_last_row_is_decode(lib):
    """The last row of each chunk sits at the context's end: it equals the decode of
    that row over the whole context."""
    bs, hq, hkv, d = 4, 8, 2, 16
    lens, tl = [21, 7, 30], [5, 7, 1]
    for dt in DTYPES:
        _, _, kc, vc, tables, ctx, qs, q = _chunk_case(600, lens, tl, hq, hkv, d, bs, dt)
        got = oracle.paged_attention_chunk(q, kc, vc, tables, ctx, qs, 0.25, lib=lib)
        last = (qs[1:] - 1).long()
        want = oracle.paged_attention(q[last].contiguous(), kc, vc, tables, ctx, 0.25, lib=lib)
        _close(got[last.numpy()], want, 0.0, f"last rows {dt}")


# ----------------------------------------------------------------------------- swap
def pin_swap_roundtrip(lib):
    """Swapping blocks out to a host pool and back in to other GPU blocks: the host pool
    receives exactly torch's indexed copy of the source blocks, every other block of
    both pools is unchanged, and the blocks swapped back in equal the originals (bf16
    bit patterns, including NaN payloads, and 8-bit codes)."""
    g = torch.Generator().manual_seed(91)
    for dt, shape in ((torch.bfloat16, (20, 2, 4, 8)), (torch.uint8, (13, 3, 16, 16))):
        if dt == torch.uint8:
            gpu = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
        else:
            gpu = torch.randn(shape, generator=g).to(dt)
            gpu.view(torch.int16)[3, 0, 0, 0] = 0x7FC1      # a NaN payload travels as bits
        host = torch.zeros((7,) + shape[1:], dtype=dt)
        out_pairs = torch.tensor([[3, 0], [11, 4], [5, 6], [0, 2]], dtype=torch.int32)
        host2 = oracle.swap_blocks(host, gpu, out_pairs, lib=lib)
        want = host.clone()
        want[out_pairs[:, 1].long()] = gpu[out_pairs[:, 0].long()]
        assert torch.equal(host2.view(torch.uint8), want.view(torch.uint8)), f"swap out {dt}"
        in_pairs = torch.tensor([[0, 9], [4, 1], [6, 12], [2, 7]], dtype=torch.int32)
        gpu2 = oracle.swap_blocks(gpu, host2, in_pairs, lib=lib)
        for (src, mid), (_, back) in zip(out_pairs.tolist(), in_pairs.tolist()):
            assert torch.equal(gpu2[back].view(torch.uint8), gpu[src].view(torch.uint8))
        keep = torch.ones(shape[0], dtype=torch.bool)
        keep[in_pairs[:, 1].long()] = False
        assert torch.equal(gpu2[keep].view(torch.uint8), gpu[keep].view(torch.uint8))
    bad = torch.tensor([[0, 7]], dtype=torch.int32)                 # outside the host pool
    try:
        oracle.swap_blocks(torch.zeros(7, 4), torch.zeros(9, 4), bad, lib=lib)
        raise AssertionError("an index outside the pool must be rejected")
    except ValueError:
        pass


ALL_PINS = [pin_decoders, pin_sdpa_library, pin_dense_bruteforce, pin_worked_example,
            pin_two_token_closed_form, pin_context_one, pin_uniform_scores, pin_zero_context,
            pin_placement_permutation, pin_gqa_equals_repeated_mha, pin_stale_slots_unread,
            pin_linearity_in_values, pin_append_roundtrip, pin_copy_on_write,
            pin_decode_step_slots, pin_fp8_decode, pin_fp8_quantize, pin_fp8_attention,
            pin_fp8_append, pin_chunk_causal_sdpa, pin_chunk_dense, pin_chunk_causality,
            pin_chunk_last_row_is_decode, pin_swap_roundtrip]
