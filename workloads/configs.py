"""Seeded synthetic decode workloads.

Each builder returns the inputs of one decode step over a paged KV cache: the
query, the K and V block pools, the block tables, the context lengths and the
softmax scale, plus (where the workload has them) the new tokens to append with
their slot mapping and the block-copy pairs of copy-on-write. Nothing here
computes attention; placement comes from :mod:`workloads.blockmgr`.

Value recipe (shared by every workload): float32 draws from N(0, 1) with a seeded
``torch.Generator``, then cast to the KV dtype (round to nearest even). The whole
pool is filled, used or not. Physical placement: a seeded random permutation of
the pool is the free-list order, so consecutive logical blocks land on scattered
physical blocks.

The shapes follow the serving workloads the pages talk about (grouped-query
heads, head_dim 128, block_size 16, variable context lengths); each builder's
docstring gives its exact recipe. Random numbers for large pools can be drawn on
the GPU (``gen_device``) so that multi-GiB pools are not generated on the host;
block tables and lengths always come from a CPU generator.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

from .blockmgr import (BlockPool, Sequence_, append_token, blocks_needed, pack_tables,
                       prefill)


@dataclass
class DecodeStep:
    """All tensors of one decode step (plus optional append and copy work)."""

    name: str
    q: Optional[torch.Tensor]                 # [B, Hq, D]
    k_cache: Optional[torch.Tensor]           # [num_blocks, Hkv, bs, D]
    v_cache: Optional[torch.Tensor]           # [num_blocks, Hkv, bs, D]
    block_tables: torch.Tensor                # int32 [B, max_blocks], -1 padded
    context_lens: torch.Tensor                # int32 [B]
    scale: float                              # an exact float32 value
    block_size: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: torch.dtype
    # optional append work (reshape_and_cache) that precedes the decode
    new_k: Optional[torch.Tensor] = None      # [T, Hkv, D]
    new_v: Optional[torch.Tensor] = None
    slot_mapping: Optional[torch.Tensor] = None   # int64 [T]
    # optional copy-on-write block copies that precede the append
    copy_pairs: Optional[torch.Tensor] = None     # int32 [n, 2] (src, dst)
    # context lengths before the append (for the pre-append decode of the tiny case)
    context_lens_before: Optional[torch.Tensor] = None
    block_tables_before: Optional[torch.Tensor] = None
    partition_size: int = 0
    # 8-bit caches: k_cache/v_cache hold OCP FP8 E4M3 codes (uint8) with these scales
    kv_scales: Optional[Tuple[float, float]] = None
    # several query tokens per sequence: q is [num_query_tokens, Hq, D] and sequence b
    # owns rows query_start[b] .. query_start[b+1]-1 (its last context tokens)
    query_start: Optional[torch.Tensor] = None    # int32 [B + 1]
    max_query_len: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.numel())

    @property
    def num_blocks(self) -> int:
        return int(self.extra["num_blocks"])

    def kv_bytes(self) -> int:
        """Bytes of K and V one decode step reads: sum(ctx) * Hkv * 2 * D * elt, with
        elt the cache element size (1 for 8-bit caches)."""
        elt = 1 if self.kv_scales is not None else \
            torch.empty((), dtype=self.dtype).element_size()
        return int(self.context_lens.to(torch.int64).sum()) * self.num_kv_heads * 2 \
            * self.head_dim * elt


def fp32_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) rounded to float32 (both sides receive this exact value)."""
    return float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32))


def _normal(shape, dtype, gen: torch.Generator, device) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    return x.to(dtype)


def _gens(seed: int, gen_device) -> Tuple[torch.Generator, torch.Generator]:
    """A CPU generator for structure and one on ``gen_device`` for values."""
    g_cpu = torch.Generator(device="cpu").manual_seed(seed)
    dev = torch.device(gen_device)
    g_val = g_cpu if dev.type == "cpu" else torch.Generator(device=dev).manual_seed(seed)
    return g_cpu, g_val


def _fill_pools(num_blocks, hkv, bs, d, dtype, g_val, gen_device, device, materialize):
    if not materialize:
        return None, None
    k = _normal((num_blocks, hkv, bs, d), dtype, g_val, gen_device).to(device)
    v = _normal((num_blocks, hkv, bs, d), dtype, g_val, gen_device).to(device)
    return k, v


def tiny_fp32(seed: int = 1001, device="cpu", gen_device="cpu",
              materialize: bool = True) -> DecodeStep:
    """4 sequences, context lengths {7, 16, 33, 100}, block_size 4, 8 query heads =
    8 KV heads, head_dim 64, float32, a pool of 64 physical blocks; plus one append
    of 4 new tokens and one copy of 3 block pairs."""
    B, H, HKV, D, BS, NP = 4, 8, 8, 64, 4, 64
    ctx = [7, 16, 33, 100]
    g_cpu, g_val = _gens(seed, gen_device)
    perm = torch.randperm(NP, generator=g_cpu).tolist()
    pool = BlockPool(NP, perm)
    seqs = [prefill(pool, n, BS) for n in ctx]
    width = blocks_needed(max(ctx) + 1, BS)
    tables_before = torch.tensor(pack_tables(seqs, width), dtype=torch.int32)
    ctx_before = torch.tensor(ctx, dtype=torch.int32)
    slots = [append_token(pool, s, BS) for s in seqs]
    tables = torch.tensor(pack_tables(seqs, width), dtype=torch.int32)
    ctx_after = torch.tensor([s.num_tokens for s in seqs], dtype=torch.int32)
    used = sorted({b for s in seqs for b in s.table})
    free = sorted(set(range(NP)) - set(used))
    pick = torch.randperm(len(used), generator=g_cpu)[:3].tolist()
    pick_dst = torch.randperm(len(free), generator=g_cpu)[:3].tolist()
    pairs = torch.tensor([[used[i], free[j]] for i, j in zip(pick, pick_dst)],
                         dtype=torch.int32)
    q = _normal((B, H, D), torch.float32, g_val, gen_device).to(device) if materialize else None
    kc, vc = _fill_pools(NP, HKV, BS, D, torch.float32, g_val, gen_device, device, materialize)
    nk = _normal((B, HKV, D), torch.float32, g_val, gen_device).to(device) if materialize else None
    nv = _normal((B, HKV, D), torch.float32, g_val, gen_device).to(device) if materialize else None
    return DecodeStep(
        name="tiny_fp32", q=q, k_cache=kc, v_cache=vc,
        block_tables=tables.to(device), context_lens=ctx_after.to(device),
        scale=fp32_scale(D), block_size=BS, num_heads=H, num_kv_heads=HKV, head_dim=D,
        dtype=torch.float32, new_k=nk, new_v=nv,
        slot_mapping=torch.tensor(slots, dtype=torch.int64).to(device),
        copy_pairs=pairs.to(device), context_lens_before=ctx_before.to(device),
        block_tables_before=tables_before.to(device),
        extra={"num_blocks": NP, "seed": seed})


def _scattered_batch(name, seed, ctx: List[int], num_blocks: int, hq, hkv, d, bs, width,
                     dtype, device, gen_device, materialize, partition_size=0):
    g_cpu, g_val = _gens(seed, gen_device)
    perm = torch.randperm(num_blocks, generator=g_cpu).tolist()
    pool = BlockPool(num_blocks, perm)
    seqs = [prefill(pool, n, bs) for n in ctx]
    tables = torch.tensor(pack_tables(seqs, width), dtype=torch.int32)
    q = _normal((len(ctx), hq, d), dtype, g_val, gen_device).to(device) if materialize else None
    kc, vc = _fill_pools(num_blocks, hkv, bs, d, dtype, g_val, gen_device, device, materialize)
    return DecodeStep(
        name=name, q=q, k_cache=kc, v_cache=vc, block_tables=tables.to(device),
        context_lens=torch.tensor(ctx, dtype=torch.int32).to(device), scale=fp32_scale(d),
        block_size=bs, num_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
        partition_size=partition_size,
        extra={"num_blocks": num_blocks, "seed": seed})


def llama3_8b_decode(seed: int = 1002, device="cpu", gen_device=None,
                     materialize: bool = True, batch: int = 64) -> DecodeStep:
    """Llama-3-8B-shaped single-layer decode: 64 sequences, 32 query / 8 KV heads,
    head_dim 128, block_size 16, context lengths uniform in [128, 2048], blocks drawn
    from a shuffled pool of 16384, bfloat16."""
    gen_device = device if gen_device is None else gen_device
    g = torch.Generator(device="cpu").manual_seed(seed + 7919)
    ctx = torch.randint(128, 2049, (batch,), generator=g).tolist()
    return _scattered_batch("llama3_8b_decode", seed, ctx, 16384, 32, 8, 128, 16, 128,
                            torch.bfloat16, device, gen_device, materialize)


def llama_70b_decode(seed: int = 1003, device="cpu", gen_device=None,
                     materialize: bool = True) -> DecodeStep:
    """70B-shaped decode batch on one GPU: 256 sequences, 64 query / 8 KV heads,
    head_dim 128, block_size 16, context lengths log-normal (median 1024, sigma 0.8)
    clipped to [16, 4096], a shuffled pool sized to 1.1x the blocks in use, bfloat16."""
    gen_device = device if gen_device is None else gen_device
    g = torch.Generator(device="cpu").manual_seed(seed + 7919)
    z = torch.randn(256, generator=g, dtype=torch.float64)
    ctx = torch.exp(math.log(1024.0) + 0.8 * z).round().clamp(16, 4096).to(torch.int64).tolist()
    need = sum(blocks_needed(n, 16) for n in ctx)
    return _scattered_batch("llama_70b_decode", seed, ctx, math.ceil(1.1 * need), 64, 8, 128,
                            16, 256, torch.bfloat16, device, gen_device, materialize)


def skewed_decode(seed: int = 1007, device="cpu", gen_device=None,
                  materialize: bool = True) -> DecodeStep:
    """Llama-3-8B-shaped batch with one long context among short ones: 64 sequences,
    one of 4096 tokens at a seeded position and 63 uniform in [128, 512], 32 query /
    8 KV heads, head_dim 128, block_size 16, blocks drawn from a shuffled pool of
    16384, bfloat16. The long sequence holds about a sixth of the batch's KV bytes,
    which a split of one workgroup per (sequence, KV head) cannot spread."""
    gen_device = device if gen_device is None else gen_device
    g = torch.Generator(device="cpu").manual_seed(seed + 7919)
    ctx = torch.randint(128, 513, (64,), generator=g).tolist()
    ctx[int(torch.randint(0, 64, (1,), generator=g))] = 4096
    return _scattered_batch("skewed_decode", seed, ctx, 16384, 32, 8, 128, 16, 256,
                            torch.bfloat16, device, gen_device, materialize)


def long_context_decode(seed: int = 1004, device="cpu", gen_device=None,
                        materialize: bool = True) -> DecodeStep:
    """Long-context decode for the split-K path: 8 sequences, 32 query / 8 KV heads,
    head_dim 128, block_size 16, context lengths uniform in [32768, 131072], shuffled
    pool of 1.1x the blocks in use, bfloat16, partitions of 512 tokens."""
    gen_device = device if gen_device is None else gen_device
    g = torch.Generator(device="cpu").manual_seed(seed + 7919)
    ctx = torch.randint(32768, 131073, (8,), generator=g).tolist()
    need = sum(blocks_needed(n, 16) for n in ctx)
    return _scattered_batch("long_context_decode", seed, ctx, math.ceil(1.1 * need), 32, 8,
                            128, 16, 8192, torch.bfloat16, device, gen_device, materialize,
                            partition_size=512)


def shared_prefix_cow(seed: int = 1005, device="cpu", gen_device=None,
                      materialize: bool = True, prefix_tokens: int = 2048,
                      prompts: int = 32, samples: int = 8) -> DecodeStep:
    """Parallel sampling over shared prompts: 32 prompts x 8 samples (256 sequences),
    each prompt's prefix stored once and referenced by all its samples, 1-256
    divergent tokens per sample, 32 query / 8 KV heads, head_dim 128, block_size 16,
    bfloat16.

    Order of device work in the step: copy the last prefix block for every sample
    but the first (copy_blocks, K and V pools), write every token placed after the
    fork (the divergent tokens and the new one) with reshape_and_cache, then decode
    with context = prefix + divergent + 1.

    With ``prefix_tokens=2048`` the prefix fills its 128 blocks exactly, so the
    first divergent token opens a fresh block; the last prefix block is still
    copied for samples 1..7 before the first divergent write (the literal reading
    of the workload's recipe). With a prefix that ends mid-block (e.g. 2040) the
    copy is the genuine copy-on-write: the first divergent write lands in the
    shared, partly filled block.
    """
    gen_device = device if gen_device is None else gen_device
    BS, HQ, HKV, D = 16, 32, 8, 128
    g_cpu, g_val = _gens(seed, gen_device)
    g_len = torch.Generator(device="cpu").manual_seed(seed + 7919)
    div = torch.randint(1, 257, (prompts * samples,), generator=g_len).tolist()
    nb_prefix = blocks_needed(prefix_tokens, BS)
    need = prompts * nb_prefix + prompts * (samples - 1) + sum(
        blocks_needed(prefix_tokens + d + 1, BS) - nb_prefix + 1 for d in div)
    num_blocks = math.ceil(1.1 * need)
    perm = torch.randperm(num_blocks, generator=g_cpu).tolist()
    pool = BlockPool(num_blocks, perm)
    copies: List[Tuple[int, int]] = []
    seqs: List[Sequence_] = []
    for p in range(prompts):
        root = prefill(pool, prefix_tokens, BS)
        group = [root] + [root.copy_shared(pool) for _ in range(samples - 1)]
        last = nb_prefix - 1
        if prefix_tokens % BS == 0:
            # full last block: copy it explicitly for samples 1.. (literal recipe)
            for s in group[1:]:
                old = s.table[last]
                new = pool.allocate(1)[0]
                copies.append((old, new))
                pool.decref(old)
                s.table[last] = new
        seqs.extend(group)
    slots: List[int] = []
    for s, d in zip(seqs, div):
        for _ in range(d + 1):  # divergent tokens, then the new token
            slots.append(append_token(pool, s, BS, copies))
    width = max(len(s.table) for s in seqs)
    tables = torch.tensor(pack_tables(seqs, width), dtype=torch.int32)
    ctx = torch.tensor([s.num_tokens for s in seqs], dtype=torch.int32)
    T = len(slots)
    q = _normal((len(seqs), HQ, D), torch.bfloat16, g_val, gen_device).to(device) \
        if materialize else None
    kc, vc = _fill_pools(num_blocks, HKV, BS, D, torch.bfloat16, g_val, gen_device, device,
                         materialize)
    nk = _normal((T, HKV, D), torch.bfloat16, g_val, gen_device).to(device) if materialize else None
    nv = _normal((T, HKV, D), torch.bfloat16, g_val, gen_device).to(device) if materialize else None
    return DecodeStep(
        name="shared_prefix_cow" if prefix_tokens % BS == 0 else "shared_prefix_cow_partial",
        q=q, k_cache=kc, v_cache=vc, block_tables=tables.to(device),
        context_lens=ctx.to(device), scale=fp32_scale(D), block_size=BS, num_heads=HQ,
        num_kv_heads=HKV, head_dim=D, dtype=torch.bfloat16, new_k=nk, new_v=nv,
        slot_mapping=torch.tensor(slots, dtype=torch.int64).to(device),
        copy_pairs=torch.tensor(copies, dtype=torch.int32).reshape(-1, 2).to(device),
        extra={"num_blocks": num_blocks, "seed": seed, "prefix_tokens": prefix_tokens,
               "divergent": div, "samples": samples, "prompts": prompts})


def random_small(seed: int, *, batch: int, num_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, max_ctx: int, dtype=torch.float32, min_ctx: int = 1,
                 num_blocks: Optional[int] = None, device="cpu",
                 gen_device="cpu") -> DecodeStep:
    """A small random batch (for brute-force and parity sweeps): lengths uniform in
    [min_ctx, max_ctx], blocks scattered over a shuffled pool with some spare."""
    g = torch.Generator(device="cpu").manual_seed(seed + 7919)
    ctx = torch.randint(min_ctx, max_ctx + 1, (batch,), generator=g).tolist()
    need = sum(blocks_needed(n, block_size) for n in ctx)
    nb = num_blocks if num_blocks is not None else need + 3 + need // 4
    width = max(1, max(blocks_needed(n, block_size) for n in ctx))
    return _scattered_batch(f"random_small_{seed}", seed, ctx, nb, num_heads, num_kv_heads,
                            head_dim, block_size, width, dtype, device, gen_device, True)


def batch_with_lengths(seed: int, lens: List[int], *, num_heads: int, num_kv_heads: int,
                       head_dim: int, block_size: int, dtype=torch.float32, spare: int = 5,
                       device="cpu", gen_device="cpu") -> DecodeStep:
    """A batch with exactly these context lengths (edge-case tests), blocks scattered
    over a shuffled pool with ``spare`` unused blocks."""
    need = sum(blocks_needed(n, block_size) for n in lens)
    width = max(1, max(blocks_needed(n, block_size) for n in lens))
    return _scattered_batch(f"lengths_{seed}", seed, list(lens), need + spare, num_heads,
                            num_kv_heads, head_dim, block_size, width, dtype, device,
                            gen_device, True)


def llama3_8b_decode_fp8(seed: int = 1002, device="cpu", gen_device=None,
                         materialize: bool = True) -> DecodeStep:
    """The Llama-3-8B-shaped batch with 8-bit (E4M3) caches, scales FP8_SCALES."""
    return with_fp8(llama3_8b_decode(seed, device, gen_device, materialize))




FP8_SCALES = (0.0137, 0.0211)


def with_fp8(step: DecodeStep, scales: Tuple[float, float] = FP8_SCALES) -> DecodeStep:
    """8-bit copy of a batch's caches: each pool value x becomes the OCP FP8 E4M3 code of
    clamp(x / scale, -448, 448) through torch's float8_e4m3fn conversion, so the cache
    holds scale * E4M3(...) (inputs only; the library's own quantising append is tested
    separately). With N(0, 1) values and scales near 1/73 the codes span most of the
    E4M3 range. q and any rows to append keep their dtype."""
    def codes(x, scale):
        y = (x.float() / scale).clamp_(-448.0, 448.0)
        return y.to(torch.float8_e4m3fn).view(torch.uint8)
    step.k_cache = codes(step.k_cache, scales[0])
    step.v_cache = codes(step.v_cache, scales[1])
    step.kv_scales = (float(scales[0]), float(scales[1]))
    step.name = step.name + "_fp8"
    return step


def with_chunk(step: DecodeStep, query_lens: List[int], seed: int = 0) -> DecodeStep:
    """Turn a batch into a multi-token query step: sequence b's last query_lens[b]
    context tokens become its query rows (a prefill chunk or draft tokens to verify;
    their K/V are the pool's values at those positions). q is redrawn as
    [sum(query_lens), Hq, D] from N(0, 1), cast to the KV dtype (bf16/f16 for 8-bit
    caches: the dtype of the batch)."""
    if len(query_lens) != step.num_seqs:
        raise ValueError("one query length per sequence")
    dev = step.context_lens.device
    qs = [0]
    for n in query_lens:
        qs.append(qs[-1] + int(n))
    gen = torch.Generator(device=dev).manual_seed(seed + 15485863)
    step.q = _normal((qs[-1], step.num_heads, step.head_dim), step.dtype, gen, dev)
    step.query_start = torch.tensor(qs, dtype=torch.int32).to(dev)
    step.max_query_len = max(query_lens) if query_lens else 0
    # the chunk tokens' own K/V rows and slots (positions n - T .. n - 1), for a step
    # that appends them before attending
    tables = step.block_tables.to("cpu")
    bs = step.block_size
    slots = []
    for b, (n, T) in enumerate(zip(step.context_lens.to("cpu").tolist(), query_lens)):
        for pos in range(n - T, n):
            slots.append(int(tables[b, pos // bs]) * bs + pos % bs if pos >= 0 else -1)
    shape = (qs[-1], step.num_kv_heads, step.head_dim)
    step.new_k = _normal(shape, step.dtype, gen, dev)
    step.new_v = _normal(shape, step.dtype, gen, dev)
    step.slot_mapping = torch.tensor(slots, dtype=torch.int64).to(dev)
    step.name = step.name + "_chunk"
    return step


def llama3_8b_verify4(seed: int = 1002, device="cpu", gen_device=None,
                      materialize: bool = True) -> DecodeStep:
    """Draft verification on the Llama-3-8B-shaped batch: each sequence's last 4
    context tokens are queries (speculative decoding checks 4 draft tokens at once)."""
    s = llama3_8b_decode(seed, device, gen_device, materialize)
    s = with_chunk(s, [4] * s.num_seqs, seed=seed)
    s.name = "llama3_8b_verify4"
    return s


def prefill_chunk512(seed: int = 1006, device="cpu", gen_device=None,
                     materialize: bool = True) -> DecodeStep:
    """Chunked prefill: 8 sequences, 32/8 heads, D 128, bs 16, bf16; contexts
    U[1024, 4096] whose last 512 tokens are the chunk being prefilled (each attends the
    earlier tokens and the chunk up to itself). Pool = 1.1 x the blocks in use."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    ctx = torch.randint(1024, 4097, (8,), generator=g).tolist()
    need = sum(blocks_needed(n, 16) for n in ctx)
    nb = int(math.ceil(1.1 * need))
    width = max(blocks_needed(n, 16) for n in ctx)
    s = _scattered_batch("prefill_chunk512", seed, ctx, nb, 32, 8, 128, 16, width,
                         torch.bfloat16, device, gen_device or device, materialize)
    s = with_chunk(s, [512] * len(ctx), seed=seed)
    s.name = "prefill_chunk512"
    return s


def with_shared_prefixes(step: DecodeStep, sizes: List[int],
                         prefixes: List[int]) -> DecodeStep:
    """Make groups of consecutive sequences share prefix blocks: group i holds the next
    sizes[i] sequences, and its members' first prefixes[i] table entries are set to its
    first member's entries (the samples of one prompt pointing at the prompt's blocks).
    The members' own blocks at those positions are simply no longer referenced. A
    member shorter than the prefix keeps only its own length. The groups are stored as
    step.extra["group_start"] / ["group_prefix"] (lists)."""
    if sum(sizes) != step.num_seqs or len(prefixes) != len(sizes):
        raise ValueError("group sizes must cover the batch, one prefix per group")
    tables = step.block_tables.to("cpu").clone()
    width = tables.shape[1]
    start = [0]
    for k, p in zip(sizes, prefixes):
        a = start[-1]
        if p > width:
            raise ValueError("prefix longer than the table rows")
        if p > 0 and int(tables[a, p - 1]) < 0:
            raise ValueError("a group's first member must hold the whole prefix")
        tables[a + 1:a + k, :p] = tables[a, :p]
        start.append(a + k)
    step.block_tables = tables.to(step.block_tables.device)
    step.extra["group_start"] = start
    step.extra["group_prefix"] = list(prefixes)
    return step


def with_append(step: DecodeStep, seed: int = 0) -> DecodeStep:
    """Turn a decode batch into a full decode step: the last token of every context
    is the newly generated one, so its K/V are written into its slot first
    (reshape_and_cache) and the decode then attends to it. New K/V values are drawn
    like everything else (float32 N(0, 1), cast to the KV dtype); the slot of the
    token at position ctx-1 is table[(ctx-1) // bs] * bs + (ctx-1) % bs."""
    if step.new_k is not None:
        return step
    tables = step.block_tables.to("cpu")
    ctx = step.context_lens.to("cpu").tolist()
    bs = step.block_size
    slots = []
    for b, n in enumerate(ctx):
        if n <= 0:
            slots.append(-1)
            continue
        pos = n - 1
        slots.append(int(tables[b, pos // bs]) * bs + pos % bs)
    dev = step.block_tables.device
    gen = torch.Generator(device=dev).manual_seed(seed + 104729)
    shape = (len(ctx), step.num_kv_heads, step.head_dim)
    step.new_k = _normal(shape, step.dtype, gen, dev)
    step.new_v = _normal(shape, step.dtype, gen, dev)
    step.slot_mapping = torch.tensor(slots, dtype=torch.int64).to(dev)
    return step


WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "llama3_8b_decode": llama3_8b_decode,
    "llama3_8b_decode_fp8": llama3_8b_decode_fp8,
    "llama3_8b_verify4": llama3_8b_verify4,
    "prefill_chunk512": prefill_chunk512,
    "llama_70b_decode": llama_70b_decode,
    "long_context_decode": long_context_decode,
    "shared_prefix_cow": shared_prefix_cow,
    "skewed_decode": skewed_decode,
}
