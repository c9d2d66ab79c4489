"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Bars: bit-exact for reshape_and_cache and copy_blocks (whole pools compared, the
untouched bytes included); attention within max-abs 1e-5 for float32 KV and 2e-2
for bfloat16 KV (float32 accumulation). float16 KV uses 5e-3: its 10-bit mantissa
rounds the output 8x finer than bfloat16's 7 bits, so the bfloat16 bound scaled by
that ratio is 2.5e-3; 5e-3 leaves a 2x margin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_374_amd as pkv
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 5e-3}
DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _max_err(got, want):
    g = got.detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - want))) if g.size else 0.0


def decode(s, q=None, kc=None, vc=None, tables=None, ctx=None, partition_size=0):
    q = s.q if q is None else q
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode(out, q, s.k_cache if kc is None else kc,
                               s.v_cache if vc is None else vc,
                               s.block_tables if tables is None else tables,
                               s.context_lens if ctx is None else ctx, s.scale,
                               partition_size=partition_size)
    torch.cuda.synchronize()
    return out


def oracle_decode(s, rows=None, kc=None, vc=None, ctx=None, tables=None):
    return oracle.paged_attention(s.q, s.k_cache if kc is None else kc,
                                  s.v_cache if vc is None else vc,
                                  s.block_tables if tables is None else tables,
                                  s.context_lens if ctx is None else ctx, s.scale, rows=rows)


# ------------------------------------------------------------------ tiny float32 case
def test_tiny_fp32_full_step():
    _say("tiny_fp32: decode, copy_blocks, reshape_and_cache, decode")
    s = W.tiny_fp32(device=DEV, gen_device="cpu")
    out0 = decode(s, ctx=s.context_lens_before, tables=s.block_tables_before)
    want0 = oracle_decode(s, ctx=s.context_lens_before, tables=s.block_tables_before)
    assert _max_err(out0, want0) <= TOL[torch.float32]
    kc, vc = s.k_cache.clone(), s.v_cache.clone()
    pkv.copy_blocks([kc, vc], s.copy_pairs)
    torch.cuda.synchronize()
    ek = oracle.copy_blocks(s.k_cache, s.copy_pairs)
    ev = oracle.copy_blocks(s.v_cache, s.copy_pairs)
    assert torch.equal(kc.cpu(), ek) and torch.equal(vc.cpu(), ev)
    pkv.reshape_and_cache(s.new_k, s.new_v, kc, vc, s.slot_mapping)
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(s.new_k, s.new_v, ek, ev, s.slot_mapping)
    assert torch.equal(kc.cpu(), ek) and torch.equal(vc.cpu(), ev)
    out1 = decode(s, kc=kc, vc=vc)
    want1 = oracle_decode(s, kc=ek, vc=ev)
    assert _max_err(out1, want1) <= TOL[torch.float32]
    for part in (4, 8, 16, 64):          # forced split-K through the reduction kernel
        outp = decode(s, kc=kc, vc=vc, partition_size=part)
        assert _max_err(outp, want1) <= TOL[torch.float32], part


# ------------------------------------------------------------------ random sweep
SWEEP = []
for dt in (torch.float32, torch.bfloat16, torch.float16):
    for d in (64, 128, 256):
        for bs, g in ((1, 1), (2, 2), (4, 4), (8, 8), (16, 1), (16, 4), (16, 8), (32, 2)):
            SWEEP.append((dt, d, bs, g))


@pytest.mark.parametrize("dt,d,bs,group", SWEEP,
                         ids=[f"{str(a).split('.')[-1]}-d{b}-bs{c}-g{e}" for a, b, c, e in SWEEP])
def test_random_batches(dt, d, bs, group):
    seed = 300 + d + bs * 7 + group * 13 + TOL[dt].__hash__() % 17
    _say(f"random batch {dt} d={d} bs={bs} g={group} seed={seed}")
    s = W.random_small(seed, batch=5, num_heads=2 * group, num_kv_heads=2, head_dim=d,
                       block_size=bs, max_ctx=600, min_ctx=1, dtype=dt, device=DEV)
    want = oracle_decode(s)
    for part in (0, 64 if bs <= 64 else bs):
        part = (part // bs) * bs
        out = decode(s, partition_size=part)
        err = _max_err(out, want)
        assert err <= TOL[dt], f"partition {part}: max err {err}"


def test_ragged_edges_bf16():
    """Lengths at 1, block boundaries +-1 and a partition boundary, one empty row."""
    _say("ragged edges bf16")
    lens = [1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 0, 1024]
    s = W.random_small(77, batch=len(lens), num_heads=8, num_kv_heads=2, head_dim=128,
                       block_size=16, max_ctx=1024, dtype=torch.bfloat16, device=DEV)
    ctx = torch.tensor(lens, dtype=torch.int32)
    # rebuild tables for these lengths from a fresh shuffled pool
    pool = W.BlockPool(s.num_blocks, torch.randperm(s.num_blocks,
                                                    generator=torch.Generator().manual_seed(3)))
    seqs = [W.prefill(pool, n, 16) for n in lens]
    tables = torch.tensor(W.pack_tables(seqs, 64), dtype=torch.int32)
    s.block_tables, s.context_lens = tables.to(DEV), ctx.to(DEV)
    want = oracle_decode(s)
    for part in (0, 512, 16):
        out = decode(s, partition_size=part)
        assert torch.all(out[10].float() == 0), "empty context must give zeros"
        assert _max_err(out, want) <= TOL[torch.bfloat16], part


# ------------------------------------------------------------------ invariants
def test_context_one_returns_v0_bit_exact():
    for dt in (torch.float32, torch.bfloat16):
        _say(f"ctx=1 {dt}")
        s = W.random_small(88, batch=4, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                           max_ctx=1, dtype=dt, device=DEV)
        out = decode(s)
        tb = s.block_tables.cpu()
        for b in range(4):
            for h in range(8):
                v0 = s.v_cache[int(tb[b, 0]), h // 4, 0]
                assert torch.equal(out[b, h], v0), (b, h)


def test_placement_permutation_bit_identical():
    _say("placement permutation bf16")
    s = W.random_small(91, batch=6, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       max_ctx=900, dtype=torch.bfloat16, device=DEV)
    perm = torch.randperm(s.num_blocks, generator=torch.Generator().manual_seed(5)).to(DEV)
    kc2 = torch.empty_like(s.k_cache)
    vc2 = torch.empty_like(s.v_cache)
    kc2[perm] = s.k_cache
    vc2[perm] = s.v_cache
    tb = s.block_tables.clone()
    used = tb >= 0
    tb[used] = perm[tb[used].long()].to(torch.int32)
    a = decode(s)
    b = decode(s, kc=kc2, vc=vc2, tables=tb)
    assert torch.equal(a, b)


def test_stale_slots_and_free_blocks_poisoned_with_nan():
    _say("NaN poisoning bf16 and fp32")
    for dt in (torch.bfloat16, torch.float32):
        s = W.random_small(93, batch=6, num_heads=8, num_kv_heads=2, head_dim=128,
                           block_size=16, max_ctx=500, dtype=dt, device=DEV)
        a = decode(s)
        kc, vc = s.k_cache.clone(), s.v_cache.clone()
        tb, ctx = s.block_tables.cpu(), s.context_lens.cpu()
        keep = torch.zeros(s.num_blocks, 16, dtype=torch.bool)
        for b in range(tb.shape[0]):
            for t in range(int(ctx[b])):
                keep[int(tb[b, t // 16]), t % 16] = True
        poison = (~keep).to(DEV)
        kc.permute(0, 2, 1, 3)[poison] = float("nan")
        vc.permute(0, 2, 1, 3)[poison] = float("nan")
        for part in (0, 64):
            b2 = decode(s, kc=kc, vc=vc, partition_size=part)
            a2 = a if part == 0 else decode(s, partition_size=part)
            assert torch.equal(a2, b2), (dt, part)


def test_deterministic_across_runs():
    _say("determinism")
    s = W.random_small(95, batch=8, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       max_ctx=2000, dtype=torch.bfloat16, device=DEV)
    assert torch.equal(decode(s), decode(s))
    assert torch.equal(decode(s, partition_size=256), decode(s, partition_size=256))


# ------------------------------------------------------------------ serving-shape workloads
def _fused_full(s, part, label):
    """The fused step (append at each context end, then attend) on a whole workload:
    both pools byte for byte against the oracle's append, the whole output against
    the oracle's decode over those pools."""
    W.with_append(s, seed=int(s.extra["seed"]))
    kc0, vc0 = s.k_cache, s.v_cache
    want, ek, ev = oracle.decode_step(s.q, s.new_k, s.new_v, kc0, vc0, s.block_tables,
                                      s.context_lens, s.scale)
    kc, vc = kc0.clone(), vc0.clone()
    out = torch.full_like(s.q, float("nan"))
    pkv.paged_attention_decode_append(out, s.q, s.new_k, s.new_v, kc, vc, s.block_tables,
                                      s.context_lens, s.scale, partition_size=part)
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu(), ek), f"{label}: K pool differs from the oracle's append"
    assert torch.equal(vc.cpu(), ev), f"{label}: V pool differs from the oracle's append"
    err = _max_err(out, want)
    _say(f"  {label} fused step partition {part}: max err {err:.3e}")
    assert err <= TOL[torch.bfloat16], f"{label} fused partition {part}: max err {err}"


def test_llama3_8b_decode_full():
    _say("llama3_8b_decode: full output vs oracle")
    s = W.llama3_8b_decode(device=DEV, gen_device=DEV)
    want = oracle_decode(s)
    out = decode(s)
    assert _max_err(out, want) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("reps", [8, 10], ids=["512-units-paired", "640-units-longest-first"])
def test_per_unit_path_ragged_lengths(reps):
    """At least 512 (sequence, KV head) units with table rows of at most 256 blocks take
    one workgroup per unit (a workspace of the counters plus piece records for 64
    helpers and one per sequence per KV head suffices on that path, and is far too
    small for the balanced path's): 512 units pair long
    contexts with short ones on a CU, more run longest first. Ragged lengths with empty
    contexts, one-token contexts and block-edge tails: full output against the oracle,
    deterministic, and the fused step bit-identical to the two-call form, caches byte
    for byte."""
    lens = [0, 1, 15, 16, 17, 100, 513, 2048, 2047, 33, 1024, 7, 300, 1500, 64, 65] * reps
    _say(f"per-unit path: {len(lens)} sequences x 4 KV heads")
    s = W.batch_with_lengths(2900, lens, num_heads=16, num_kv_heads=4, head_dim=128,
                             block_size=16, dtype=torch.bfloat16, device=DEV)
    width = s.block_tables.shape[1]
    assert width <= 256
    record = (4 * 128 + 2 * 4 + 63) // 64 * 64 * 4
    need = (1 << 20) + 4 * (64 + len(lens)) * record
    assert pkv.workspace_size(len(lens), 16, 4, 128, 16, width, 0) >= need
    # through the C call with a workspace of exactly that size
    lib = pkv.load()
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    out0 = torch.full_like(s.q, float("nan"))
    rc = lib.pkv_paged_attention_decode(
        out0.data_ptr(), s.q.data_ptr(), s.k_cache.data_ptr(), s.v_cache.data_ptr(),
        s.block_tables.data_ptr(), s.context_lens.data_ptr(), float(s.scale), len(lens), 16,
        4, 128, 16, width, s.k_cache.shape[0], 1, 0, ws.data_ptr(), need,
        torch.cuda.current_stream(DEV).cuda_stream)
    assert rc == 0, pkv.strerror(rc)
    out = decode(s)
    assert torch.equal(out, out0)
    assert _max_err(out, oracle_decode(s)) <= TOL[torch.bfloat16]
    assert torch.equal(out, decode(s)), "deterministic"
    W.with_append(s, seed=2900)
    kc_a, vc_a = s.k_cache.clone(), s.v_cache.clone()
    kc_b, vc_b = s.k_cache.clone(), s.v_cache.clone()
    out_a, out_b = torch.empty_like(s.q), torch.empty_like(s.q)
    pkv.paged_attention_decode_append(out_a, s.q, s.new_k, s.new_v, kc_a, vc_a, s.block_tables,
                                      s.context_lens, s.scale)
    pkv.reshape_and_cache(s.new_k, s.new_v, kc_b, vc_b, s.slot_mapping)
    pkv.paged_attention_decode(out_b, s.q, kc_b, vc_b, s.block_tables, s.context_lens,
                               s.scale)
    torch.cuda.synchronize()
    assert torch.equal(kc_a, kc_b) and torch.equal(vc_a, vc_b), "fused append differs"
    assert torch.equal(out_a, out_b), "fused step != two calls"


def test_per_unit_remembered_ranks():
    """The per-unit form remembers, per lengths buffer, which sequence held each position
    of the longest-first order, and checks the guess exactly before using it. Repeated
    calls on one buffer (guesses right), lengths rewritten in place so that the order
    changes (guesses wrong, the search runs again), and the call after that: every output
    against the oracle, repeated calls bit-identical."""
    lens = [0, 1, 15, 16, 17, 100, 513, 2048, 2047, 33, 1024, 7, 300, 1500, 64, 65] * 8
    _say(f"remembered ranks: {len(lens)} sequences x 4 KV heads")
    s = W.batch_with_lengths(2911, lens, num_heads=16, num_kv_heads=4, head_dim=128,
                             block_size=16, dtype=torch.bfloat16, device=DEV)
    assert s.block_tables.shape[1] <= 256
    first = decode(s)
    assert _max_err(first, oracle_decode(s)) <= TOL[torch.bfloat16]
    for _ in range(2):
        assert torch.equal(decode(s), first), "a repeated call differs"
    # new lengths in the same buffer, each within its row's blocks: the order changes
    rng = np.random.default_rng(2911)
    new = [int(rng.integers(0, n + 1)) for n in lens]
    s.context_lens.copy_(torch.tensor(new, dtype=torch.int32, device=DEV))
    second = decode(s)
    assert _max_err(second, oracle_decode(s)) <= TOL[torch.bfloat16]
    assert torch.equal(decode(s), second), "a repeated call differs"


def test_llama_70b_decode_full():
    """70B-shaped batch (256 sequences, 64/8 heads, log-normal contexts up to 4096):
    every output row against the oracle on the library's own split (one workgroup per
    unit, longest first) and on 512-token partitions plus the reduction; then the
    fused step on the library's split."""
    _say("llama_70b_decode: full output vs oracle")
    s = W.llama_70b_decode(device=DEV, gen_device=DEV)
    want = oracle_decode(s)
    for part in (0, 512):
        err = _max_err(decode(s, partition_size=part), want)
        _say(f"  partition {part}: max err {err:.3e}")
        assert err <= TOL[torch.bfloat16], f"partition {part}: max err {err}"
    _fused_full(s, 0, "llama_70b_decode")


def test_skewed_decode_full():
    """One 4096-token context among 63 of 128-512 tokens: every output row against the
    oracle on the library's own split and on 512-token partitions plus the reduction;
    then the fused step on the library's split."""
    _say("skewed_decode: full output vs oracle")
    s = W.skewed_decode(device=DEV, gen_device=DEV)
    want = oracle_decode(s)
    for part in (0, 512):
        err = _max_err(decode(s, partition_size=part), want)
        _say(f"  partition {part}: max err {err:.3e}")
        assert err <= TOL[torch.bfloat16], f"partition {part}: max err {err}"
    _fused_full(s, 0, "skewed_decode")


def test_long_context_split_k_full():
    """Long contexts (8 sequences, 32K-128K tokens): every output row against the
    oracle with 512-token partitions plus the reduction, and on the library's own
    split (equal shares merged across workgroups); then the fused step with 512-token
    partitions."""
    _say("long_context_decode: full output vs oracle")
    s = W.long_context_decode(device=DEV, gen_device=DEV)
    want = oracle_decode(s)
    for part in (512, 0):
        err = _max_err(decode(s, partition_size=part), want)
        _say(f"  partition {part}: max err {err:.3e}")
        assert err <= TOL[torch.bfloat16], f"partition {part}: max err {err}"
    _fused_full(s, 512, "long_context_decode")


REDUCE = [(torch.float32, 64, 32), (torch.float32, 256, 32), (torch.bfloat16, 128, 16),
          (torch.float16, 64, 16)]


@pytest.mark.parametrize("dt,d,part", REDUCE,
                         ids=[f"{str(a).split('.')[-1]}-d{b}-p{c}" for a, b, c in REDUCE])
def test_reduce_many_partitions(dt, d, part):
    """Contexts cut into hundreds of partitions (up to 512), one empty row and one
    single-partition row: the reduction kernel against the oracle."""
    _say(f"reduce over many partitions {dt} d={d} partition={part}")
    lens = [8192, 5000, 0, part, 7777, 1]
    s = W.batch_with_lengths(1200 + d + part, lens, num_heads=8, num_kv_heads=2, head_dim=d,
                             block_size=16, dtype=dt, device=DEV)
    want = oracle_decode(s)
    out = decode(s, partition_size=part)
    assert torch.all(out[2].float() == 0), "empty context must give zeros"
    assert _max_err(out, want) <= TOL[dt]


@pytest.mark.parametrize("prefix", [2048, 2040, 40])
def test_shared_prefix_cow_step(prefix):
    """The shared-prefix batch in the pages' order: copy-on-write copies, every token
    placed after the fork written, then the decode. Pools byte for byte; every output
    row against the oracle on the library's split and on 512-token partitions. Then
    the same step with the newest token appended by the fused call.

    With 2048 and 2040 prefix tokens the lengths lie within an eighth of the longest
    (the kernel keeps the batch order); with 40 they span 42..297 (it ranks them):
    both orders read the shared blocks with the cache policy for shared blocks."""
    _say(f"shared_prefix_cow prefix={prefix}: copy_blocks, reshape_and_cache, decode")
    s = W.shared_prefix_cow(device=DEV, gen_device=DEV, prefix_tokens=prefix)
    kc, vc = s.k_cache.clone(), s.v_cache.clone()
    if prefix == 2048:
        pkv.copy_blocks([kc, vc], s.copy_pairs)
    else:                                   # the prepared form of the same call
        pkv.PreparedCopyBlocks([kc, vc], s.copy_pairs)()
    pkv.reshape_and_cache(s.new_k, s.new_v, kc, vc, s.slot_mapping)
    torch.cuda.synchronize()
    ek = oracle.copy_blocks(s.k_cache, s.copy_pairs)
    ev = oracle.copy_blocks(s.v_cache, s.copy_pairs)
    ek, ev = oracle.reshape_and_cache(s.new_k, s.new_v, ek, ev, s.slot_mapping)
    assert torch.equal(kc.cpu(), ek) and torch.equal(vc.cpu(), ev)
    want = oracle_decode(s, kc=ek, vc=ev)
    for part in (0, 512):
        err = _max_err(decode(s, kc=kc, vc=vc, partition_size=part), want)
        _say(f"  partition {part}: max err {err:.3e}")
        assert err <= TOL[torch.bfloat16], f"partition {part}: max err {err}"
    # fused form: each sequence's newest token is the last of its slots; write the
    # others with reshape_and_cache, then append the newest and attend in one call
    B = s.num_seqs
    last = torch.cumsum(torch.tensor([d + 1 for d in s.extra["divergent"]]), 0) - 1
    rest = torch.ones(s.slot_mapping.numel(), dtype=torch.bool)
    rest[last] = False
    kc2, vc2 = s.k_cache.clone(), s.v_cache.clone()
    pkv.copy_blocks([kc2, vc2], s.copy_pairs)
    pkv.reshape_and_cache(s.new_k[rest.to(DEV)].contiguous(), s.new_v[rest.to(DEV)].contiguous(),
                          kc2, vc2, s.slot_mapping[rest.to(DEV)].contiguous())
    out = torch.full_like(s.q, float("nan"))
    lastd = last.to(DEV)
    pkv.paged_attention_decode_append(out, s.q, s.new_k[lastd].contiguous(),
                                      s.new_v[lastd].contiguous(), kc2, vc2, s.block_tables,
                                      s.context_lens, s.scale)
    torch.cuda.synchronize()
    assert last.numel() == B
    assert torch.equal(kc2.cpu(), ek) and torch.equal(vc2.cpu(), ev), "fused append differs"
    err = _max_err(out, want)
    _say(f"  fused step: max err {err:.3e}")
    assert err <= TOL[torch.bfloat16], f"fused step: max err {err}"


def _prompt_major_identical_q(s):
    """q with every sample of a prompt given the first sample's query rows."""
    P, S = s.extra["prompts"], s.extra["samples"]
    q = s.q.view(P, S, s.num_heads, s.head_dim)
    return q[:, :1].expand(P, S, s.num_heads, s.head_dim).contiguous().view_as(s.q)


def test_shared_prefix_identical_contributions():
    """Samples of one prompt point at the same physical prefix blocks. With identical
    queries:
      * attending only the shared prefix gives bit-identical output rows for the 8
        samples, before and after copy-on-write (the copied block holds the same
        bytes at another address), on the library's split and on 512-token
        partitions, and the rows match the oracle;
      * on the whole contexts with 512-token partitions, the records of the four
        prefix partitions (tokens 0..2047) are bit-identical across the samples;
      * with the suffix made identical too (same length, same bytes in each sample's
        private blocks), the whole outputs are bit-identical."""
    _say("shared prefix: identical prefix contributions (prefix 2048, 32 x 8 samples)")
    s = W.shared_prefix_cow(device=DEV, gen_device=DEV, prefix_tokens=2048)
    P, S, H, D = s.extra["prompts"], s.extra["samples"], s.num_heads, s.head_dim
    q = _prompt_major_identical_q(s)
    kc, vc = s.k_cache.clone(), s.v_cache.clone()
    tables_before = s.block_tables.clone()
    # before the copy: samples 1..7 still point at the root's block 127
    for src, dst in s.copy_pairs.tolist():
        tables_before[tables_before == dst] = src
    pkv.copy_blocks([kc, vc], s.copy_pairs)
    pkv.reshape_and_cache(s.new_k, s.new_v, kc, vc, s.slot_mapping)
    torch.cuda.synchronize()
    prefix_ctx = torch.full_like(s.context_lens, 2048)
    want = oracle.paged_attention(q, kc, vc, s.block_tables, prefix_ctx, s.scale)
    for tables, label in ((tables_before, "shared block 127"), (s.block_tables, "after CoW")):
        for part in (0, 512):
            out = torch.full_like(q, float("nan"))
            pkv.paged_attention_decode(out, q, kc, vc, tables, prefix_ctx, s.scale,
                                       partition_size=part)
            torch.cuda.synchronize()
            o = out.view(P, S, H, D)
            assert torch.equal(o, o[:, :1].expand_as(o)), f"{label} partition {part}"
            assert _max_err(out, want) <= TOL[torch.bfloat16], f"{label} partition {part}"
    # prefix partition records on the whole contexts
    B, MB = s.num_seqs, s.block_tables.shape[1]
    npart, (om, ol, oo) = pkv.partials_layout(B, H, s.num_kv_heads, D, 16, MB, 512,
                                              torch.bfloat16)
    assert npart == (MB * 16 + 511) // 512 and npart >= 5
    ws = torch.zeros(pkv.workspace_size(B, H, s.num_kv_heads, D, 16, MB, 512),
                     dtype=torch.uint8, device=DEV)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode(out, q, kc, vc, s.block_tables, s.context_lens, s.scale,
                               partition_size=512, workspace=ws)
    torch.cuda.synchronize()
    rows = B * H * npart
    m = ws[om:om + rows * 4].view(torch.float32).view(P, S, H, npart)[..., :4]
    l = ws[ol:ol + rows * 4].view(torch.float32).view(P, S, H, npart)[..., :4]
    o = ws[oo:oo + rows * D * 4].view(torch.float32).view(P, S, H, npart, D)[..., :4, :]
    for name, x in (("m", m), ("l", l), ("o", o)):
        assert torch.all(torch.isfinite(x)), name
        assert torch.equal(x, x[:, :1].expand_as(x)), f"prefix partition records {name}"
    assert torch.all(l >= 1.0), "every prefix partition holds its reference token"
    # identical suffixes: every sample of a prompt attends the prompt's shortest
    # context, and each sample's private blocks get the first sample's bytes
    ctx = s.context_lens.view(P, S).min(dim=1, keepdim=True).values.expand(P, S)
    ctx = ctx.contiguous().view(-1)
    tb = s.block_tables.cpu().view(P, S, MB)
    src_ids, dst_ids = [], []
    for p_, n in enumerate(ctx.view(P, S)[:, 0].tolist()):
        for j in range(128, (n + 15) // 16):
            for s_ in range(1, S):
                src_ids.append(int(tb[p_, 0, j]))
                dst_ids.append(int(tb[p_, s_, j]))
    assert min(src_ids + dst_ids) >= 0 and len(set(dst_ids)) == len(dst_ids)
    src_t = torch.tensor(src_ids, device=DEV)
    dst_t = torch.tensor(dst_ids, device=DEV)
    kc[dst_t] = kc[src_t]
    vc[dst_t] = vc[src_t]
    for part in (0, 512):
        out = torch.full_like(q, float("nan"))
        pkv.paged_attention_decode(out, q, kc, vc, s.block_tables, ctx, s.scale,
                                   partition_size=part)
        torch.cuda.synchronize()
        o = out.view(P, S, H, D)
        assert torch.equal(o, o[:, :1].expand_as(o)), f"identical suffix partition {part}"
    want = oracle.paged_attention(q, kc, vc, s.block_tables, ctx, s.scale)
    assert _max_err(out, want) <= TOL[torch.bfloat16]


# ------------------------------------------------------------------ matrix-core paths
BAL = [(dt, hq, hkv, batch, max_ctx)
       for dt in (torch.bfloat16, torch.float16)
       for hq, hkv, batch, max_ctx in ((8, 8, 3, 40), (8, 4, 7, 300), (12, 4, 5, 1000),
                                       (32, 8, 64, 2048), (40, 8, 9, 700), (64, 8, 33, 1500),
                                       (32, 2, 4, 5000), (16, 1, 1, 20000), (4, 1, 300, 64))]


@pytest.mark.parametrize("dt,hq,hkv,batch,max_ctx", BAL,
                         ids=[f"{str(a).split('.')[-1]}-h{b}-kv{c}-B{d}-ctx{e}"
                              for a, b, c, d, e in BAL])
def test_mfma_balanced_and_partitioned(dt, hq, hkv, batch, max_ctx):
    """Shares of a few blocks (many units cut between workgroups, merged by the last
    one to finish), groups 1..16, and the fixed-partition kernel plus reduction."""
    seed = 500 + hq + 3 * hkv + 7 * batch + max_ctx % 97
    _say(f"mfma {dt} hq={hq} hkv={hkv} batch={batch} max_ctx={max_ctx} seed={seed}")
    s = W.random_small(seed, batch=batch, num_heads=hq, num_kv_heads=hkv, head_dim=128,
                       block_size=16, max_ctx=max_ctx, min_ctx=1, dtype=dt, device=DEV)
    want = oracle_decode(s)
    for part in (0, 512, 16):
        out = decode(s, partition_size=part)
        err = _max_err(out, want)
        assert err <= TOL[dt], f"partition {part}: max err {err}"
    # the balanced path leaves its counters zeroed: a second call agrees bit for bit
    assert torch.equal(decode(s), decode(s))


def test_mfma_empty_and_short_rows():
    _say("mfma: empty rows mixed with one-token and block-boundary rows")
    lens = [0, 1, 16, 0, 17, 2048, 0, 31, 33, 0]
    s = W.random_small(611, batch=len(lens), num_heads=32, num_kv_heads=8, head_dim=128,
                       block_size=16, max_ctx=2048, dtype=torch.bfloat16, device=DEV)
    pool = W.BlockPool(s.num_blocks, torch.randperm(s.num_blocks,
                                                    generator=torch.Generator().manual_seed(9)))
    seqs = [W.prefill(pool, n, 16) for n in lens]
    s.block_tables = torch.tensor(W.pack_tables(seqs, 128), dtype=torch.int32).to(DEV)
    s.context_lens = torch.tensor(lens, dtype=torch.int32).to(DEV)
    want = oracle_decode(s)
    for part in (0, 512):
        out = decode(s, partition_size=part)
        for b, n in enumerate(lens):
            if n == 0:
                assert torch.all(out[b].float() == 0), (part, b)
        assert _max_err(out, want) <= TOL[torch.bfloat16], part
    allzero = torch.zeros_like(s.context_lens)
    out = decode(s, ctx=allzero)
    assert torch.all(out.float() == 0)


def test_one_workspace_shared_by_every_path():
    """A fixed-partition call must not disturb the balanced path's merge counters when
    both use one workspace (regression: scratch used to overlap the counters)."""
    _say("shared workspace: partitioned, balanced, generic, balanced")
    s = W.random_small(701, batch=16, num_heads=32, num_kv_heads=8, head_dim=128,
                       block_size=16, max_ctx=3000, dtype=torch.bfloat16, device=DEV)
    MB = s.block_tables.shape[1]
    need = max(pkv.workspace_size(16, 32, 8, 128, 16, MB, p) for p in (0, 512, 16))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    pkv.workspace_init(ws)
    want = oracle_decode(s)
    outs = []
    for part in (512, 0, 16, 0, 0):
        out = torch.full_like(s.q, float("nan"))
        pkv.paged_attention_decode(out, s.q, s.k_cache, s.v_cache, s.block_tables,
                                   s.context_lens, s.scale, partition_size=part, workspace=ws)
        torch.cuda.synchronize()
        assert _max_err(out, want) <= TOL[torch.bfloat16], part
        outs.append(out)
    assert torch.equal(outs[1], outs[3]) and torch.equal(outs[3], outs[4])


def test_prepared_calls_and_graph_replays():
    """The prepared-call API and HIP-graph replays of it give the eager results on
    every replay, with eager work and synchronisations between replays."""
    _say("prepared calls + graph replays")
    s = W.random_small(703, batch=24, num_heads=32, num_kv_heads=8, head_dim=128,
                       block_size=16, max_ctx=2048, dtype=torch.bfloat16, device=DEV)
    W.with_append(s, seed=703)
    ref_k, ref_v = s.k_cache.clone(), s.v_cache.clone()
    pkv.reshape_and_cache(s.new_k, s.new_v, ref_k, ref_v, s.slot_mapping)
    ref = torch.empty_like(s.q)
    pkv.paged_attention_decode(ref, s.q, ref_k, ref_v, s.block_tables, s.context_lens, s.scale)
    torch.cuda.synchronize()
    out = torch.full_like(s.q, float("nan"))
    app = pkv.PreparedReshapeAndCache(s.new_k, s.new_v, s.k_cache, s.v_cache, s.slot_mapping)
    dec = pkv.PreparedDecode(out, s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                             s.scale)
    app()
    dec()
    torch.cuda.synchronize()
    assert torch.equal(s.k_cache, ref_k) and torch.equal(s.v_cache, ref_v)
    assert torch.equal(out, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        app()
        dec()
    for i in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        assert torch.equal(s.k_cache, ref_k), i


@pytest.mark.parametrize("hq,hkv,batch,max_ctx", [(32, 8, 6, 300), (16, 1, 2, 9000)])
def test_balanced_merge_never_reads_stale_partials(hq, hkv, batch, max_ctx):
    """Two batches of one shape alternate for many calls; every share is a few blocks,
    so most units are merged across workgroups from partial slots that the previous
    call filled with the other batch's data. Any stale read changes the output."""
    _say(f"stale-partial stress hq={hq} hkv={hkv} batch={batch} max_ctx={max_ctx}")
    sets = [W.random_small(800 + i, batch=batch, num_heads=hq, num_kv_heads=hkv, head_dim=128,
                           block_size=16, max_ctx=max_ctx, min_ctx=max_ctx // 2,
                           dtype=torch.bfloat16, device=DEV) for i in range(2)]
    refs, decs = [], []
    for s in sets:
        want = oracle_decode(s)
        out = torch.empty_like(s.q)
        d = pkv.PreparedDecode(out, s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                               s.scale)
        d()
        torch.cuda.synchronize()
        assert _max_err(out, want) <= TOL[torch.bfloat16]
        refs.append(out.clone())
        decs.append(d)
    for it in range(300):
        decs[it % 2]()
        if it % 2 == 1:
            torch.cuda.synchronize()
            assert torch.equal(decs[0].out, refs[0]) and torch.equal(decs[1].out, refs[1]), it
