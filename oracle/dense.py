"""Brute-force dense attention over gathered blocks (NumPy, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the definition written the other way round from the C walk: first undo
the paging (gather every used block of a sequence, in table order, into one
contiguous [context, head_dim] K and V per KV head, [P2] "Block Table 数据结构"),
then evaluate ordinary softmax attention of the single query over all of it
([P3] "PagedAttention：逻辑连续，物理不必连续": the query attends to every earlier
token and itself). Grouped-query heads are expanded by repeating each KV head for
its group. Values are widened to float64 by torch's own dtype conversion, which is
independent of the C decoder.
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def dense_attention(q, k_cache, v_cache, block_tables, context_lens, scale) -> np.ndarray:
    """[B, Hq, D] float64 outputs; zero rows for zero-length contexts."""
    qd = _f64(q)
    kd, vd = _f64(k_cache), _f64(v_cache)
    tables = block_tables.detach().to("cpu").numpy()
    ctx = context_lens.detach().to("cpu").numpy()
    B, Hq, D = qd.shape
    _, Hkv, bs, _ = kd.shape
    group = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(ctx[b])
        if n == 0:
            continue
        nb = -(-n // bs)
        ids = tables[b, :nb].astype(np.int64)
        # [nb, Hkv, bs, D] -> [Hkv, nb*bs, D] -> keep the first n tokens
        K = kd[ids].transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :n]
        V = vd[ids].transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :n]
        K = np.repeat(K, group, axis=0)            # [Hq, n, D]
        V = np.repeat(V, group, axis=0)
        s = np.einsum("hd,hnd->hn", qd[b], K) * float(scale)
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w /= w.sum(axis=1, keepdims=True)
        out[b] = np.einsum("hn,hnd->hd", w, V)
    return out


def dense_chunk_attention(q, k_cache, v_cache, block_tables, context_lens, query_start,
                          scale) -> np.ndarray:
    """Several query tokens per sequence, written as masked dense attention: gather the
    sequence's whole context into contiguous K/V, score all its query rows against all
    tokens at once, and mask with a -inf matrix whose row j keeps the tokens at
    positions <= ctx - T + j (the query at position i sees tokens 1..i). Rows that keep
    no token are zero. [NQ, Hq, D] float64."""
    qd = _f64(q)
    kd, vd = _f64(k_cache), _f64(v_cache)
    tables = block_tables.detach().to("cpu").numpy()
    ctx = context_lens.detach().to("cpu").numpy()
    qs = query_start.detach().to("cpu").numpy()
    NQ, Hq, D = qd.shape
    _, Hkv, bs, _ = kd.shape
    group = Hq // Hkv
    out = np.zeros((NQ, Hq, D), dtype=np.float64)
    for b in range(len(ctx)):
        n, r0, r1 = int(ctx[b]), int(qs[b]), int(qs[b + 1])
        T = r1 - r0
        if n == 0 or T == 0:
            continue
        nb = -(-n // bs)
        ids = tables[b, :nb].astype(np.int64)
        K = kd[ids].transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :n]
        V = vd[ids].transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :n]
        K = np.repeat(K, group, axis=0)                            # [Hq, n, D]
        V = np.repeat(V, group, axis=0)
        Q = qd[r0:r1].transpose(1, 0, 2)                           # [Hq, T, D]
        s = np.einsum("htd,hnd->htn", Q, K) * float(scale)
        pos = np.arange(n)[None, :]
        last = (n - T + np.arange(T))[:, None]                     # position of row j
        s = np.where(pos <= last, s, -np.inf)
        keep = np.isfinite(s).any(axis=2, keepdims=True)           # [Hq, T, 1]
        s = np.where(keep, s - np.where(keep, s.max(axis=2, keepdims=True), 0.0), -np.inf)
        w = np.exp(s)
        den = w.sum(axis=2, keepdims=True)
        w = np.where(keep, w / np.where(keep, den, 1.0), 0.0)
        out[r0:r1] = np.einsum("htn,hnd->htd", w, V).transpose(1, 0, 2)
    return out
