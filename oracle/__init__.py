"""Independent CPU reference ("oracle") for paged decode attention and its companions.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product library
never loads it, and the two share no code: the only thing both sides use is the
seeded input generator in :mod:`workloads`.

Two implementations live here:
  * ``oracle.c`` (loaded through ctypes): the fp64 token-by-token walk of the
    block table, two-pass softmax, OpenMP over (sequence, query head); plus the
    slot-mapped append and the whole-block copy. This is the reference the GPU
    results are compared with.
  * :mod:`oracle.dense` (NumPy, fp64): gather each sequence's blocks into a
    contiguous K/V, then softmax(q K^T * scale) V. A brute-force cross-check of
    the C walk on small inputs.
Both are pinned by the CPU test-suite to things other than themselves: the
worked example of the pages, closed forms, invariants, a library attention
routine, and planted mistakes that must fail.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

from .dense import dense_attention, dense_chunk_attention  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
FP8 = 3   # uint8 tensors holding OCP FP8 E4M3 codes

_P = ctypes.c_void_p
_I = ctypes.c_int


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    lib.oracle_paged_attention.restype = _I
    lib.oracle_paged_attention.argtypes = [_P, _P, _P, _P, _I, _P, _P, ctypes.c_double, _I, _I,
                                           _I, _I, _I, _I, _I, _P, _I, _I]
    lib.oracle_reshape_and_cache.restype = _I
    lib.oracle_reshape_and_cache.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I]
    lib.oracle_copy_blocks.restype = _I
    lib.oracle_copy_blocks.argtypes = [_P, _P, _I, _I, ctypes.c_long]
    lib.oracle_decode.restype = _I
    lib.oracle_decode.argtypes = [_P, _P, ctypes.c_long, _I]
    lib.oracle_quantize_fp8.restype = _I
    lib.oracle_quantize_fp8.argtypes = [_P, _P, ctypes.c_long, _I, ctypes.c_float]
    lib.oracle_paged_attention_kv.restype = _I
    lib.oracle_paged_attention_kv.argtypes = [_P, _P, _I, _P, _P, _I, ctypes.c_double,
                                              ctypes.c_double, _P, _P, ctypes.c_double, _I,
                                              _I, _I, _I, _I, _I, _I, _P, _I, _I]
    lib.oracle_paged_attention_chunk.restype = _I
    lib.oracle_paged_attention_chunk.argtypes = [_P, _P, _I, _P, _P, _I, ctypes.c_double,
                                                 ctypes.c_double, _P, _P, _P, ctypes.c_double,
                                                 _I, _I, _I, _I, _I, _I, _I, _I, _I]
    lib.oracle_reshape_and_cache_fp8.restype = _I
    lib.oracle_reshape_and_cache_fp8.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                                 ctypes.c_float, ctypes.c_float]
    lib.oracle_swap_blocks.restype = _I
    lib.oracle_swap_blocks.argtypes = [_P, _P, _P, _I, _I, _I, ctypes.c_long]
    lib.oracle_max_threads.restype = _I
    return lib


def _raw(t: torch.Tensor) -> np.ndarray:
    """Host bytes of a tensor as a contiguous NumPy array (bf16/f16 as raw int16)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    return t.numpy()


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def decode(t: torch.Tensor, lib=None) -> np.ndarray:
    """Element values of a float32/bfloat16/float16 tensor as float64 (C decoder)."""
    lib = lib or _load()
    raw = _raw(t)
    out = np.empty(raw.size, dtype=np.float64)
    rc = lib.oracle_decode(_ptr(out), _ptr(raw), raw.size, DTYPE_CODE[t.dtype])
    if rc != 0:
        raise ValueError(f"oracle_decode failed ({rc})")
    return out.reshape(tuple(t.shape))


def paged_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                    rows: Optional[Sequence[Tuple[int, int]]] = None, threads: int = 0,
                    lib=None) -> np.ndarray:
    """fp64 paged decode attention. Returns [B, Hq, D], or [len(rows), D] for the
    (sequence, head) pairs in ``rows``."""
    lib = lib or _load()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,Hq,D] and caches [num_blocks,Hkv,bs,D]")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q and caches must share a dtype")
    B, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    if D2 != D:
        raise ValueError("head_dim mismatch")
    qa, ka, va = _raw(q), _raw(k_cache), _raw(v_cache)
    tables = np.ascontiguousarray(block_tables.to("cpu", torch.int32).numpy())
    ctx = np.ascontiguousarray(context_lens.to("cpu", torch.int32).numpy())
    mb = tables.shape[1] if tables.ndim == 2 else 0
    if rows is not None:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        out = np.zeros((r.shape[0], D), dtype=np.float64)
        rp, nr = _ptr(r), r.shape[0]
    else:
        out = np.zeros((B, Hq, D), dtype=np.float64)
        rp, nr = None, 0
    rc = lib.oracle_paged_attention(_ptr(out), _ptr(qa), _ptr(ka), _ptr(va),
                                    DTYPE_CODE[q.dtype], _ptr(tables), _ptr(ctx),
                                    float(scale), B, Hq, Hkv, D, bs, mb, NB, rp, nr,
                                    int(threads))
    if rc != 0:
        raise ValueError(f"oracle_paged_attention rejected its inputs ({rc})")
    return out


class PreparedAttention:
    """Host copies of one decode step's inputs, marshalled once, so that repeated
    oracle evaluations (the benchmark's CPU baseline) time only the C walk."""

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, scale, lib=None,
                 kv_scales: Optional[Tuple[float, float]] = None):
        self.lib = lib or _load()
        B, Hq, D = q.shape
        NB, Hkv, bs, _ = k_cache.shape
        self.dims = (B, Hq, Hkv, D, bs, NB)
        self.dtype = DTYPE_CODE[q.dtype]
        # 8-bit caches: uint8 E4M3 codes with their two scales
        self.kv_scales = None if kv_scales is None else tuple(float(x) for x in kv_scales)
        self.qa = _raw(q)
        if self.kv_scales is None:
            self.ka, self.va = _raw(k_cache), _raw(v_cache)
        else:
            self.ka = np.ascontiguousarray(k_cache.detach().cpu().numpy())
            self.va = np.ascontiguousarray(v_cache.detach().cpu().numpy())
        self.tables = np.ascontiguousarray(block_tables.to("cpu", torch.int32).numpy())
        self.ctx = np.ascontiguousarray(context_lens.to("cpu", torch.int32).numpy())
        self.scale = float(scale)

    def __call__(self, rows: Optional[Sequence[Tuple[int, int]]] = None,
                 threads: int = 0) -> np.ndarray:
        B, Hq, Hkv, D, bs, NB = self.dims
        mb = self.tables.shape[1] if self.tables.ndim == 2 else 0
        if rows is not None:
            r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
            out = np.zeros((r.shape[0], D), dtype=np.float64)
            rp, nr = _ptr(r), r.shape[0]
        else:
            out = np.zeros((B, Hq, D), dtype=np.float64)
            rp, nr = None, 0
        if self.kv_scales is None:
            rc = self.lib.oracle_paged_attention(_ptr(out), _ptr(self.qa), _ptr(self.ka),
                                                 _ptr(self.va), self.dtype, _ptr(self.tables),
                                                 _ptr(self.ctx), self.scale, B, Hq, Hkv, D, bs,
                                                 mb, NB, rp, nr, int(threads))
        else:
            rc = self.lib.oracle_paged_attention_kv(_ptr(out), _ptr(self.qa), self.dtype,
                                                    _ptr(self.ka), _ptr(self.va), FP8,
                                                    *self.kv_scales, _ptr(self.tables),
                                                    _ptr(self.ctx), self.scale, B, Hq, Hkv, D,
                                                    bs, mb, NB, rp, nr, int(threads))
        if rc != 0:
            raise ValueError(f"oracle_paged_attention rejected its inputs ({rc})")
        return out


# ------------------------------------------------------------------ 8-bit KV cache
def inv_scale(scale: float) -> float:
    """The binary32 reciprocal of a cache scale (one IEEE division in float32), the
    multiplier the quantising append applies."""
    return float(np.float32(1.0) / np.float32(scale))


def fp8_decode(codes: torch.Tensor, lib=None) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (a uint8 tensor) as float64 (C decoder)."""
    lib = lib or _load()
    raw = np.ascontiguousarray(codes.detach().to("cpu", torch.uint8).numpy())
    out = np.empty(raw.size, dtype=np.float64)
    if lib.oracle_decode(_ptr(out), _ptr(raw), raw.size, FP8) != 0:
        raise ValueError("oracle_decode failed")
    return out.reshape(tuple(codes.shape))


def fp8_quantize(x: torch.Tensor, inv: float, lib=None) -> torch.Tensor:
    """E4M3 codes of float32(x) * inv (binary32 product), nearest with ties to even,
    saturating at 448 (a uint8 CPU tensor shaped like x)."""
    lib = lib or _load()
    raw = _raw(x)
    out = np.empty(raw.size, dtype=np.uint8)
    if lib.oracle_quantize_fp8(_ptr(out), _ptr(raw), raw.size, DTYPE_CODE[x.dtype],
                               float(inv)) != 0:
        raise ValueError("oracle_quantize_fp8 failed")
    return torch.from_numpy(out.reshape(tuple(x.shape)))


def paged_attention_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        k_scale: float, v_scale: float, block_tables: torch.Tensor,
                        context_lens: torch.Tensor, scale: float,
                        rows: Optional[Sequence[Tuple[int, int]]] = None, threads: int = 0,
                        lib=None) -> np.ndarray:
    """fp64 paged decode attention over 8-bit caches (uint8 E4M3 codes): key =
    decode(code) * k_scale, value = decode(code) * v_scale; q in its own dtype."""
    lib = lib or _load()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,Hq,D] and caches [num_blocks,Hkv,bs,D]")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("8-bit caches are uint8 tensors of E4M3 codes")
    B, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    if D2 != D:
        raise ValueError("head_dim mismatch")
    qa = _raw(q)
    ka = np.ascontiguousarray(k_cache.detach().cpu().numpy())
    va = np.ascontiguousarray(v_cache.detach().cpu().numpy())
    tables = np.ascontiguousarray(block_tables.to("cpu", torch.int32).numpy())
    ctx = np.ascontiguousarray(context_lens.to("cpu", torch.int32).numpy())
    mb = tables.shape[1] if tables.ndim == 2 else 0
    if rows is not None:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        out = np.zeros((r.shape[0], D), dtype=np.float64)
        rp, nr = _ptr(r), r.shape[0]
    else:
        out = np.zeros((B, Hq, D), dtype=np.float64)
        rp, nr = None, 0
    rc = lib.oracle_paged_attention_kv(_ptr(out), _ptr(qa), DTYPE_CODE[q.dtype], _ptr(ka),
                                       _ptr(va), FP8, float(k_scale), float(v_scale),
                                       _ptr(tables), _ptr(ctx), float(scale), B, Hq, Hkv, D,
                                       bs, mb, NB, rp, nr, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_paged_attention_kv rejected its inputs ({rc})")
    return out


def reshape_and_cache_fp8(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float,
                          v_scale: float, lib=None):
    """Expected 8-bit pools (new uint8 CPU tensors) after the quantising append of
    k, v ([T, Hkv, D], float32/bfloat16/float16) at their slots."""
    lib = lib or _load()
    T, Hkv, D = k.shape
    NB, Hkv2, bs, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or v.shape != k.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    kc = k_cache.detach().to("cpu").clone().contiguous()
    vc = v_cache.detach().to("cpu").clone().contiguous()
    ka, va = _raw(k), _raw(v)
    kca, vca = kc.numpy(), vc.numpy()   # views of kc/vc's storage
    slots = np.ascontiguousarray(slot_mapping.to("cpu", torch.int64).numpy())
    rc = lib.oracle_reshape_and_cache_fp8(_ptr(ka), _ptr(va), _ptr(kca), _ptr(vca),
                                          _ptr(slots), T, Hkv, D, bs, NB,
                                          DTYPE_CODE[k.dtype], inv_scale(k_scale),
                                          inv_scale(v_scale))
    if rc != 0:
        raise ValueError(f"oracle_reshape_and_cache_fp8 rejected its inputs ({rc})")
    return kc, vc


def decode_step_fp8(q, new_k, new_v, k_cache, v_cache, k_scale, v_scale, block_tables,
                    context_lens, scale, lib=None):
    """decode_step over 8-bit caches: the newest tokens' rows are quantised into their
    slots, then every query attends over its whole context. Returns (out fp64, expected
    k_cache, expected v_cache)."""
    slots = context_end_slots(block_tables, context_lens, k_cache.shape[2])
    kc, vc = reshape_and_cache_fp8(new_k, new_v, k_cache, v_cache, slots, k_scale, v_scale,
                                   lib=lib)
    out = paged_attention_fp8(q, kc, vc, k_scale, v_scale, block_tables, context_lens, scale,
                              lib=lib)
    return out, kc, vc


def paged_attention_chunk(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_tables: torch.Tensor, context_lens: torch.Tensor,
                          query_start: torch.Tensor, scale: float,
                          kv_scales: Optional[Tuple[float, float]] = None, threads: int = 0,
                          lib=None) -> np.ndarray:
    """fp64 attention of several new query tokens per sequence (causal within the
    chunk): q [NQ, Hq, D]; rows query_start[b] .. query_start[b+1]-1 are the last
    tokens of sequence b, and row query_start[b] + j attends the first
    context_lens[b] - T_b + j + 1 tokens. kv_scales: 8-bit (E4M3) caches with these
    scales; otherwise the caches share q's dtype. Returns [NQ, Hq, D]."""
    lib = lib or _load()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [NQ,Hq,D] and caches [num_blocks,Hkv,bs,D]")
    NQ, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    if D2 != D:
        raise ValueError("head_dim mismatch")
    qa = _raw(q)
    if kv_scales is None:
        ka, va, kvt, ks, vs = _raw(k_cache), _raw(v_cache), DTYPE_CODE[k_cache.dtype], 1.0, 1.0
    else:
        ka = np.ascontiguousarray(k_cache.detach().cpu().numpy())
        va = np.ascontiguousarray(v_cache.detach().cpu().numpy())
        kvt, ks, vs = FP8, float(kv_scales[0]), float(kv_scales[1])
    tables = np.ascontiguousarray(block_tables.to("cpu", torch.int32).numpy())
    ctx = np.ascontiguousarray(context_lens.to("cpu", torch.int32).numpy())
    qs = np.ascontiguousarray(query_start.to("cpu", torch.int32).numpy())
    B = ctx.shape[0]
    if qs.shape != (B + 1,):
        raise ValueError("query_start must be [num_seqs + 1]")
    mb = tables.shape[1] if tables.ndim == 2 else 0
    out = np.zeros((NQ, Hq, D), dtype=np.float64)
    rc = lib.oracle_paged_attention_chunk(_ptr(out), _ptr(qa), DTYPE_CODE[q.dtype], _ptr(ka),
                                          _ptr(va), kvt, ks, vs, _ptr(tables), _ptr(ctx),
                                          _ptr(qs), float(scale), B, NQ, Hq, Hkv, D, bs, mb, NB,
                                          int(threads))
    if rc != 0:
        raise ValueError(f"oracle_paged_attention_chunk rejected its inputs ({rc})")
    return out


def reshape_and_cache(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor, lib=None):
    """Expected pools after the slot-mapped append (new CPU tensors)."""
    lib = lib or _load()
    T, Hkv, D = k.shape
    NB, Hkv2, bs, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or v.shape != k.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    kc = k_cache.detach().to("cpu").clone().contiguous()
    vc = v_cache.detach().to("cpu").clone().contiguous()
    ka, va = _raw(k), _raw(v)
    kca, vca = _raw(kc), _raw(vc)   # views of kc/vc's storage
    slots = np.ascontiguousarray(slot_mapping.to("cpu", torch.int64).numpy())
    rc = lib.oracle_reshape_and_cache(_ptr(ka), _ptr(va), _ptr(kca), _ptr(vca), _ptr(slots), T,
                                      Hkv, D, bs, NB, k.element_size())
    if rc != 0:
        raise ValueError(f"oracle_reshape_and_cache rejected its inputs ({rc})")
    return kc, vc


def context_end_slots(block_tables: torch.Tensor, context_lens: torch.Tensor,
                      block_size: int) -> torch.Tensor:
    """Slot of each sequence's newest token, the one at position n - 1 of a context
    of n tokens. The block-table walk of [P2] section "Block Table 数据结构" gives
    logical block (n - 1) // block_size at offset (n - 1) % block_size. The slot is
    physical_block * block_size + offset, and -1 (write nothing) for an empty context.
    Plain Python over lists."""
    tables = block_tables.to("cpu").tolist()
    slots = []
    for b, n in enumerate(context_lens.to("cpu").tolist()):
        if n <= 0:
            slots.append(-1)
            continue
        pos = n - 1
        slots.append(tables[b][pos // block_size] * block_size + pos % block_size)
    return torch.tensor(slots, dtype=torch.int64)


def decode_step(q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, scale,
                lib=None):
    """One decode step in the pages' order ([P3] section "Block table：为什么它能减少
    碎片"). First the newest token's K and V go into its slot, the free slot of the
    last block or the first slot of a newly taken one. Then every query attends over
    its whole context, that token included. Returns (out fp64 [B, Hq, D], expected
    k_cache, expected v_cache)."""
    slots = context_end_slots(block_tables, context_lens, k_cache.shape[2])
    kc, vc = reshape_and_cache(new_k, new_v, k_cache, v_cache, slots, lib=lib)
    return paged_attention(q, kc, vc, block_tables, context_lens, scale, lib=lib), kc, vc


def copy_blocks(cache: torch.Tensor, pairs: torch.Tensor, lib=None) -> torch.Tensor:
    """Expected pool after copying each (src, dst) block pair (a new CPU tensor)."""
    lib = lib or _load()
    c = cache.detach().to("cpu").clone().contiguous()
    ca = _raw(c)
    p = np.ascontiguousarray(pairs.to("cpu", torch.int32).numpy().reshape(-1, 2))
    block_bytes = c[0].numel() * c.element_size() if c.shape[0] else 0
    rc = lib.oracle_copy_blocks(_ptr(ca), _ptr(p), p.shape[0], c.shape[0], block_bytes)
    if rc != 0:
        raise ValueError(f"oracle_copy_blocks rejected its inputs ({rc})")
    return c


def swap_blocks(dst_pool: torch.Tensor, src_pool: torch.Tensor, pairs: torch.Tensor,
                lib=None) -> torch.Tensor:
    """Expected destination pool after copying block src of src_pool over block dst of
    dst_pool for each (src, dst) pair (a new CPU tensor). The pools share the block
    layout [blocks, ...] and dtype; their block counts may differ."""
    lib = lib or _load()
    if dst_pool.dtype != src_pool.dtype or dst_pool.shape[1:] != src_pool.shape[1:]:
        raise ValueError("pools must share dtype and block layout")
    d = dst_pool.detach().to("cpu").clone().contiguous()
    s = src_pool.detach().to("cpu").contiguous()
    da, sa = _raw(d), _raw(s)
    p = np.ascontiguousarray(pairs.to("cpu", torch.int32).numpy().reshape(-1, 2))
    block_bytes = d[0].numel() * d.element_size() if d.shape[0] else 0
    rc = lib.oracle_swap_blocks(_ptr(da), _ptr(sa), _ptr(p), p.shape[0], s.shape[0], d.shape[0],
                                block_bytes)
    if rc != 0:
        raise ValueError(f"oracle_swap_blocks rejected its inputs ({rc})")
    return d
