"""GPU parity of multi-token query attention (prefill chunks, draft verification) against
the CPU oracle: sequence b's last T_b context tokens are queries, and the query at
position i attends tokens 0..i.

Bars: max-abs 2e-2 for bfloat16 and 5e-3 for float16 outputs, as for the decode; 8-bit
caches use the bound of their query type.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_374_amd as pkv
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float16: 5e-3}
DEV = torch.device("cuda:0")
NAN = float("nan")


def _say(msg):
    print(msg, flush=True)


def _err(got, want):
    g = got.detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - want))) if g.size else 0.0


def _chunk(seed, lens, tlens, dt, group, nkv=2, fp8=False):
    s = W.batch_with_lengths(seed, lens, num_heads=nkv * group, num_kv_heads=nkv, head_dim=128,
                             block_size=16, dtype=dt, device=DEV)
    if fp8:
        W.with_fp8(s)
    return W.with_chunk(s, tlens, seed=seed)


def _run(s, max_query_len=None):
    out = torch.full_like(s.q, NAN)
    ks, vs = s.kv_scales if s.kv_scales else (None, None)
    pkv.paged_attention_chunk(out, s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                              s.query_start, s.scale,
                              max_query_len=s.max_query_len if max_query_len is None
                              else max_query_len, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return out


def _want(s):
    return oracle.paged_attention_chunk(s.q, s.k_cache, s.v_cache, s.block_tables,
                                        s.context_lens, s.query_start, s.scale,
                                        kv_scales=s.kv_scales)


# ragged contexts and chunk lengths: single tokens, whole prompts (T = n), chunks that
# straddle block edges, an empty sequence, and more rows than tokens (rows before the
# context start are zero)
LENS = [1, 15, 16, 17, 100, 513, 0, 40, 2049, 33]
TLENS = [1, 3, 16, 17, 33, 5, 0, 45, 4, 33]
CASES = [(dt, g) for dt in (torch.bfloat16, torch.float16) for g in (1, 2, 4, 8, 16)] + \
        [(torch.bfloat16, 3), (torch.bfloat16, 6)]


@pytest.mark.parametrize("dt,group", CASES,
                         ids=[f"{str(a).split('.')[-1]}-g{b}" for a, b in CASES])
def test_chunk_matches_oracle(dt, group):
    seed = 2100 + group
    _say(f"chunk {dt} g={group} seed={seed}")
    s = _chunk(seed, LENS, TLENS, dt, group)
    out = _run(s)
    want = _want(s)
    assert _err(out, want) <= TOL[dt]
    r0 = int(s.query_start[LENS.index(40)])
    assert torch.all(out[r0:r0 + 5].float() == 0), "rows before the context must be zero"
    assert torch.equal(out, _run(s)), "deterministic"


@pytest.mark.parametrize("dt,group", CASES,
                         ids=[f"{str(a).split('.')[-1]}-g{b}" for a, b in CASES])
def test_short_chunks_match_oracle(dt, group):
    """Chunks of at most four tiles (16 / G tokens each): the launch where a
    workgroup's waves split the blocks of one tile, as for draft verification. The
    long-chunk cases above run one tile per wave."""
    tq = 16 // group
    tl = [min(x, 4 * tq) for x in TLENS]
    tl[LENS.index(40)] = min(4 * tq, 45)       # still rows before the context when tq > 10
    seed = 2150 + group
    _say(f"short chunks {dt} g={group} seed={seed} tlens={tl}")
    s = _chunk(seed, LENS, tl, dt, group)
    assert (s.max_query_len + tq - 1) // tq <= 4
    out = _run(s)
    assert _err(out, _want(s)) <= TOL[dt]
    assert torch.equal(out, _run(s)), "deterministic"


@pytest.mark.parametrize("dt,group", [(torch.bfloat16, 4), (torch.float16, 8)],
                         ids=["bf16-g4", "f16-g8"])
def test_chunk_over_fp8_caches(dt, group):
    _say(f"chunk fp8 {dt} g={group}")
    s = _chunk(2200 + group, LENS, TLENS, dt, group, fp8=True)
    assert _err(_run(s), _want(s)) <= TOL[dt]


@pytest.mark.parametrize("tlens", [[3, 300], [3, 9]], ids=["long-chunks", "short-chunks"])
def test_chunk_long_context_spans_table_windows(tlens):
    """A context of 2500 blocks (more than one staging window of tables) with a few
    query tokens, next to a 700-token context, in both launch forms."""
    _say(f"chunk long context {tlens}")
    s = _chunk(2301, [40000, 700], tlens, torch.bfloat16, 4, nkv=1)
    assert _err(_run(s), _want(s)) <= TOL[torch.bfloat16]


def test_single_token_chunks_equal_the_decode():
    """T = 1 for every sequence is the decode: both calls within tolerance of the oracle
    and of each other."""
    _say("chunk T=1 vs decode")
    lens = [5, 16, 17, 300, 1]
    s = _chunk(2401, lens, [1] * len(lens), torch.bfloat16, 4)
    got = _run(s)
    dec = torch.empty_like(s.q)
    pkv.paged_attention_decode(dec, s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                               s.scale)
    torch.cuda.synchronize()
    want = oracle.paged_attention(s.q.cpu(), s.k_cache, s.v_cache, s.block_tables,
                                  s.context_lens, s.scale)
    assert _err(got, want) <= TOL[torch.bfloat16]
    assert _err(dec, want) <= TOL[torch.bfloat16]


def test_larger_max_query_len_changes_nothing():
    """Extra tiles (max_query_len above every chunk) have no rows and exit."""
    _say("chunk max_query_len slack")
    s = _chunk(2501, [50, 9, 130], [7, 2, 20], torch.bfloat16, 4)
    assert torch.equal(_run(s), _run(s, max_query_len=64))


def test_draft_verification_on_the_8b_shape():
    """Llama-3-8B-shaped batch (64 sequences, 32/8 heads) verifying 4 draft tokens per
    sequence: sampled rows against the oracle."""
    _say("chunk 8B shape, 4 draft tokens")
    s = W.llama3_8b_decode(seed=1002, device=DEV, gen_device=DEV)
    W.with_chunk(s, [4] * s.num_seqs, seed=5)
    out = _run(s)
    g = torch.Generator().manual_seed(11)
    rows = torch.randint(0, s.q.shape[0], (24,), generator=g)
    qs = s.query_start.cpu()
    kc, vc, tables = s.k_cache.cpu(), s.v_cache.cpu(), s.block_tables.cpu()
    for r in rows.tolist():
        b = int(torch.searchsorted(qs, torch.tensor(r), right=True)) - 1
        sub_q = s.q[r:r + 1].contiguous()
        n = int(s.context_lens[b]) - (int(qs[b + 1]) - r) + 1
        want = oracle.paged_attention(sub_q.cpu(), kc, vc, tables[b:b + 1],
                                      torch.tensor([n], dtype=torch.int32), s.scale)
        assert _err(out[r:r + 1], want) <= TOL[torch.bfloat16], f"row {r}"


def test_chunk_rejects_unsupported_shapes():
    s = _chunk(2601, [20, 5], [3, 2], torch.bfloat16, 4)
    q32 = s.q.float()
    with pytest.raises(pkv.PagedKVError):      # float32 queries: no matrix-core path
        pkv.paged_attention_chunk(torch.empty_like(q32), q32, s.k_cache.float(),
                                  s.v_cache.float(), s.block_tables, s.context_lens,
                                  s.query_start, s.scale)
    with pytest.raises(ValueError):            # query_start of the wrong length
        pkv.paged_attention_chunk(torch.empty_like(s.q), s.q, s.k_cache, s.v_cache,
                                  s.block_tables, s.context_lens, s.query_start[:-1], s.scale)


def test_prepared_chunk_in_graph_replays():
    """The prepared chunk call captured in a HIP graph, replayed with new queries, matches
    eager calls every time."""
    _say("prepared chunk graph replays")
    s = _chunk(2701, [300, 41, 1000, 17], [33, 41, 6, 2], torch.bfloat16, 4)
    out = torch.empty_like(s.q)
    step = pkv.PreparedChunk(out, s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                             s.query_start, s.scale, s.max_query_len)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    gen = torch.Generator(device=DEV).manual_seed(4)
    for r in range(3):
        s.q.copy_(torch.randn(s.q.shape, generator=gen, device=DEV).to(s.q.dtype))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, _run(s)), f"replay {r}"
