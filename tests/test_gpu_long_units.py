"""GPU parity of the per-unit decode when some units are too long for one workgroup.

The per-unit grid (one workgroup per (sequence, KV head)) cuts a unit of more than
twice the blocks of an average workgroup slot (blocks x slots > 2 x the blocks of all
units; two slots per CU) into pieces of P = max(ceil(S / 2), ceil(long blocks /
helpers)) blocks, S = ceil(blocks of all units / slots): the unit's own workgroup
folds the first, helper workgroups the others, and the last piece to finish merges
them. Every case compares the whole output with the oracle (bfloat16 bound
2e-2, float16 5e-3, as in the other parity tests), checks that a second call gives the
same bits (the merge counters are left at zero), and reads the workspace to check that
the pieces were really cut where the rule above puts them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_374_amd as pkv
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float16: 5e-3}
DEV = torch.device("cuda:0")
COUNTER_BYTES = 1 << 20      # merge counters at the start of every workspace
MAX_HELPERS = 64


def _say(msg):
    print(msg, flush=True)


def _err(got, want):
    g = got.detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - want)))


def _slot_floats(group):
    gmax = 4 if group <= 4 else 8 if group <= 8 else 16
    return (gmax * 128 + 2 * gmax + 63) // 64 * 64, gmax


def _expected_pieces(lens, hkv):
    """(sequence, pieces, first record) of every cut unit, per the rule above."""
    slots = 2 * torch.cuda.get_device_properties(DEV).multi_processor_count
    helpers = min(MAX_HELPERS, max(1, slots // hkv))
    nbs = [(max(n, 0) + 15) // 16 for n in lens]
    total = sum(nbs) * hkv

    def is_long(nb):
        return nb * slots > 2 * total

    if not is_long(max(nbs)):
        return [], helpers
    S = max(1, -(-total // slots))
    long_blocks = sum(nb for nb in nbs if is_long(nb))
    P = max((S + 1) // 2, -(-long_blocks // helpers))
    cut, c = [], 0
    for b, nb in enumerate(nbs):
        if is_long(nb):
            kk = -(-nb // P)
            if kk > 1:
                cut.append((b, kk, c))
            c += kk
    return cut, helpers


def _mix(seed, n_seqs, longs, short_hi, zero_at=None):
    """n_seqs lengths uniform in [1, short_hi], with `longs` {index: length} set."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(1, short_hi + 1, (n_seqs,), generator=g).tolist()
    for i, n in longs.items():
        lens[i] = n
    if zero_at is not None:
        lens[zero_at] = 0
    return lens


# (label, seed, lengths, query heads, KV heads, dtype)
CASES = [
    ("one long, group 4", 2101, _mix(2101, 64, {18: 4096}, 512), 32, 8, torch.bfloat16),
    ("three long at both ends, group 8", 2102, _mix(2102, 64, {0: 4096, 31: 3001, 63: 2500},
                                                     200), 64, 8, torch.bfloat16),
    ("twenty long, 4 KV heads (pieces sized by the helpers)", 2103,
     _mix(2103, 128, {i: 4096 - 7 * i for i in range(3, 128, 6)}, 64, zero_at=5), 16, 4,
     torch.bfloat16),
    ("long in the upper lanes, 2 KV heads", 2104,
     _mix(2104, 256, {200: 4000, 255: 4096, 130: 2049}, 48), 4, 2, torch.float16),
    ("one long, group 16", 2105, _mix(2105, 64, {40: 4096}, 300), 128, 8, torch.bfloat16),
]


def _batch(case):
    label, seed, lens, hq, hkv, dt = case
    s = W.batch_with_lengths(seed, lens, num_heads=hq, num_kv_heads=hkv, head_dim=128,
                             block_size=16, dtype=dt, device=DEV)
    return s, lens, hkv


def _workspace(s):
    need = pkv.workspace_size(s.num_seqs, s.num_heads, s.num_kv_heads, s.head_dim,
                              s.block_size, s.block_tables.shape[1], 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    return ws


def _check_records(ws, s, lens, hkv):
    """Counters back at zero; the records of every cut unit hold finite maxima."""
    assert not torch.any(ws[:COUNTER_BYTES]), "merge counters left non-zero"
    cut, helpers = _expected_pieces(lens, hkv)
    assert cut, "the case should cut at least one unit"
    group = s.num_heads // hkv
    kf, gmax = _slot_floats(group)
    per_head = MAX_HELPERS + s.num_seqs
    rec = ws[COUNTER_BYTES:COUNTER_BYTES + hkv * per_head * kf * 4]
    rec = rec.view(torch.float32).view(hkv, per_head, kf).cpu()
    for b, kk, c in cut:
        m = rec[:, c:c + kk, gmax * 128:gmax * 128 + group]   # m of every head, piece
        assert torch.all(torch.isfinite(m)) and torch.all(m != 0), (b, kk, c)
    return cut


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_long_units_cut_into_pieces(case):
    s, lens, hkv = _batch(case)
    _say(f"long units: {case[0]} seed={case[1]}")
    want = oracle.paged_attention(s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                                  s.scale)
    ws = _workspace(s)
    outs = []
    for _ in range(2):
        out = torch.full_like(s.q, float("nan"))
        pkv.paged_attention_decode(out, s.q, s.k_cache, s.v_cache, s.block_tables,
                                   s.context_lens, s.scale, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out)
    err = _err(outs[0], want)
    _say(f"  max err {err:.3e}")
    assert err <= TOL[case[5]], err
    assert torch.equal(outs[0], outs[1]), "second call differs"
    cut = _check_records(ws, s, lens, hkv)
    _say(f"  cut units (sequence, pieces): {[(b, kk) for b, kk, _ in cut]}")


def test_long_units_fused_append():
    """The fused step on a batch with cut units: the piece holding the newest token
    writes it; pools byte for byte and outputs against the oracle."""
    s, lens, hkv = _batch(CASES[1])
    _say("long units: fused append, three long at both ends")
    W.with_append(s, seed=2102)
    want, ek, ev = oracle.decode_step(s.q, s.new_k, s.new_v, s.k_cache, s.v_cache,
                                      s.block_tables, s.context_lens, s.scale)
    kc, vc = s.k_cache.clone(), s.v_cache.clone()
    out = torch.full_like(s.q, float("nan"))
    ws = _workspace(s)
    pkv.paged_attention_decode_append(out, s.q, s.new_k, s.new_v, kc, vc, s.block_tables,
                                      s.context_lens, s.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu(), ek) and torch.equal(vc.cpu(), ev), "pools differ"
    err = _err(out, want)
    _say(f"  max err {err:.3e}")
    assert err <= TOL[torch.bfloat16], err
    _check_records(ws, s, lens, hkv)


def test_long_units_fp8():
    """8-bit caches on a batch with cut units."""
    s, lens, hkv = _batch(CASES[0])
    _say("long units: fp8 caches, one long")
    W.with_fp8(s)
    ks, vs = s.kv_scales
    want = oracle.paged_attention_fp8(s.q, s.k_cache, s.v_cache, ks, vs, s.block_tables,
                                      s.context_lens, s.scale)
    ws = _workspace(s)
    out = torch.full_like(s.q, float("nan"))
    pkv.paged_attention_decode_fp8(out, s.q, s.k_cache, s.v_cache, ks, vs, s.block_tables,
                                   s.context_lens, s.scale, workspace=ws)
    torch.cuda.synchronize()
    err = _err(out, want)
    _say(f"  max err {err:.3e}")
    assert err <= TOL[torch.bfloat16], err
    _check_records(ws, s, lens, hkv)
