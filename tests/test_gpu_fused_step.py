"""GPU parity of the fused decode step (pkv_paged_attention_decode_append).

The step is checked three ways:
  * the caches after the call equal the oracle's append at each context end, byte
    for byte (untouched slots included);
  * the output is within the attention tolerance of the oracle's decode over those
    caches;
  * the output is bit-identical to the two-call form on the GPU
    (reshape_and_cache with the context-end slots, then paged_attention_decode).
    A load that saw the stale slot instead of the new row breaks that equality:
    every pool is filled with random values, so stale rows differ from new ones.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_374_amd as pkv
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 5e-3}
DEV = torch.device("cuda:0")
NAN = float("nan")


def _say(msg):
    print(msg, flush=True)


def _err(got, want):
    g = got.detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - want))) if g.size else 0.0


def _batch(seed, lens, dt, d, bs, group, nkv=2):
    """A batch with exactly these context lengths on a shuffled pool of random values,
    plus one new K/V row per sequence."""
    s = W.batch_with_lengths(seed, lens, num_heads=nkv * group, num_kv_heads=nkv,
                             head_dim=d, block_size=bs, dtype=dt, device=DEV)
    gen = torch.Generator().manual_seed(seed + 1)
    shape = (len(lens), nkv, d)
    s.new_k = torch.randn(shape, generator=gen).to(dt).to(DEV)
    s.new_v = torch.randn(shape, generator=gen).to(dt).to(DEV)
    return s


def _two_calls(s, kc, vc, part):
    slots = oracle.context_end_slots(s.block_tables, s.context_lens, s.block_size).to(DEV)
    pkv.reshape_and_cache(s.new_k, s.new_v, kc, vc, slots)
    out = torch.full_like(s.q, NAN)
    pkv.paged_attention_decode(out, s.q, kc, vc, s.block_tables, s.context_lens, s.scale,
                               partition_size=part)
    torch.cuda.synchronize()
    return out


LENS = [1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 0, 1024, 2, 700]
CASES = [
    # dtype, head_dim, block_size, group, partition_size (0 = library's choice)
    (torch.bfloat16, 128, 16, 4, 0),     # matrix cores, balanced split
    (torch.bfloat16, 128, 16, 8, 0),
    (torch.float16, 128, 16, 16, 0),
    (torch.bfloat16, 128, 16, 1, 0),
    (torch.bfloat16, 128, 16, 4, 512),   # matrix cores, fixed partitions + reduce
    (torch.float16, 128, 16, 8, 16),
    (torch.float32, 64, 4, 2, 0),        # VALU kernel: append kernel, then decode
    (torch.bfloat16, 64, 8, 2, 0),
    (torch.float32, 128, 16, 4, 64),
]


@pytest.mark.parametrize("dt,d,bs,group,part", CASES,
                         ids=[f"{str(a).split('.')[-1]}-d{b}-bs{c}-g{e}-p{f}"
                              for a, b, c, e, f in CASES])
def test_fused_step_matches_oracle_and_two_calls(dt, d, bs, group, part):
    seed = 900 + d + bs + 7 * group + part
    _say(f"fused step {dt} d={d} bs={bs} g={group} part={part} seed={seed}")
    s = _batch(seed, LENS, dt, d, bs, group)
    kc0, vc0 = s.k_cache.clone(), s.v_cache.clone()
    want, ek, ev = oracle.decode_step(s.q, s.new_k, s.new_v, kc0, vc0, s.block_tables,
                                      s.context_lens, s.scale)
    kc, vc = kc0.clone(), vc0.clone()
    out = torch.full_like(s.q, NAN)
    pkv.paged_attention_decode_append(out, s.q, s.new_k, s.new_v, kc, vc, s.block_tables,
                                      s.context_lens, s.scale, partition_size=part)
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu(), ek), "K pool differs from the oracle's append"
    assert torch.equal(vc.cpu(), ev), "V pool differs from the oracle's append"
    assert torch.all(out[LENS.index(0)].float() == 0), "empty context must give zeros"
    err = _err(out, want)
    assert err <= TOL[dt], f"max err {err}"
    ref = _two_calls(s, kc0.clone(), vc0.clone(), part)
    assert torch.equal(out, ref), "fused step differs from append-then-decode"


def test_fused_step_context_one_is_the_new_value():
    """ctx = 1: the only token is the one being appended, so every head returns its
    V row exactly (p = 1, l = 1)."""
    _say("fused step ctx=1")
    s = _batch(41, [1] * 9, torch.bfloat16, 128, 16, 4)
    out = torch.full_like(s.q, NAN)
    pkv.paged_attention_decode_append(out, s.q, s.new_k, s.new_v, s.k_cache, s.v_cache,
                                      s.block_tables, s.context_lens, s.scale)
    torch.cuda.synchronize()
    want = s.new_v.repeat_interleave(4, dim=1)
    assert torch.equal(out, want)


def test_fused_step_repeated_rounds_on_the_8b_shape():
    """Llama-3-8B-shaped batch (64 sequences, 32/8 heads, contexts 128..2048): ten
    rounds, each appending fresh rows into the same slots. Every round the fused
    output equals the two-call output bit for bit, and the caches agree. A stale read
    would surface as a mismatch in some round. The last round is also checked
    against the oracle on sampled rows."""
    _say("fused step, 8B shape, 10 rounds")
    s = W.with_append(W.llama3_8b_decode(seed=1002, device=DEV, gen_device=DEV), seed=1002)
    kc_a, vc_a = s.k_cache.clone(), s.v_cache.clone()
    kc_b, vc_b = s.k_cache, s.v_cache
    gen = torch.Generator(device=DEV).manual_seed(5)
    out_a, out_b = torch.empty_like(s.q), torch.empty_like(s.q)
    for r in range(10):
        s.new_k = torch.randn(s.new_k.shape, generator=gen, device=DEV).to(s.dtype)
        s.new_v = torch.randn(s.new_v.shape, generator=gen, device=DEV).to(s.dtype)
        pkv.paged_attention_decode_append(out_a, s.q, s.new_k, s.new_v, kc_a, vc_a,
                                          s.block_tables, s.context_lens, s.scale)
        pkv.reshape_and_cache(s.new_k, s.new_v, kc_b, vc_b, s.slot_mapping)
        pkv.paged_attention_decode(out_b, s.q, kc_b, vc_b, s.block_tables, s.context_lens,
                                   s.scale)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), f"round {r}: fused != two calls"
    assert torch.equal(kc_a, kc_b) and torch.equal(vc_a, vc_b)
    g = torch.Generator().manual_seed(9)
    rows = [(int(b), int(h)) for b, h in zip(torch.randint(0, 64, (48,), generator=g),
                                             torch.randint(0, 32, (48,), generator=g))]
    want = oracle.paged_attention(s.q, kc_b, vc_b, s.block_tables, s.context_lens, s.scale,
                                  rows=rows)
    got = torch.stack([out_a[b, h] for b, h in rows])
    assert _err(got, want) <= TOL[torch.bfloat16]


def test_prepared_fused_step_in_a_graph():
    """The fused step bound once (PreparedDecode with new_k/new_v) and replayed from a
    HIP graph: every replay, with new rows copied in between, matches the eager
    two-call form."""
    _say("prepared fused step, graph replays")
    s = _batch(57, [300, 17, 1, 0, 1000, 64, 65], torch.bfloat16, 128, 16, 4)
    kc, vc = s.k_cache.clone(), s.v_cache.clone()
    out = torch.empty_like(s.q)
    step = pkv.PreparedDecode(out, s.q, kc, vc, s.block_tables, s.context_lens, s.scale,
                              new_k=s.new_k, new_v=s.new_v)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    gen = torch.Generator().manual_seed(3)
    kc_ref, vc_ref = s.k_cache.clone(), s.v_cache.clone()
    for r in range(6):
        s.new_k.copy_(torch.randn(s.new_k.shape, generator=gen).to(s.dtype))
        s.new_v.copy_(torch.randn(s.new_v.shape, generator=gen).to(s.dtype))
        g.replay()
        torch.cuda.synchronize()
        ref = _two_calls(s, kc_ref, vc_ref, 0)
        assert torch.equal(out, ref), f"replay {r}"
        assert torch.equal(kc, kc_ref) and torch.equal(vc, vc_ref), f"replay {r} caches"


def test_fused_step_rejects_missing_rows():
    s = _batch(61, [5, 9], torch.bfloat16, 128, 16, 4)
    out = torch.empty_like(s.q)
    with pytest.raises(ValueError):
        pkv.paged_attention_decode_append(out, s.q, s.new_k[:1], s.new_v, s.k_cache,
                                          s.v_cache, s.block_tables, s.context_lens, s.scale)
    with pytest.raises(ValueError):
        pkv.PreparedDecode(out, s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                           s.scale, new_k=s.new_k)
