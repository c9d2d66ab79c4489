"""MI355X (gfx950) paged KV-cache decode attention.

A thin binding over the C ABI of ``libpagedkv.so`` (declared in include/pagedkv.h).
The functions here only marshal arguments: every step of the computation runs in
the library's HIP kernels. PyTorch supplies device memory and the current stream.
There is no fallback: if the library is not built, or a tensor is not on a GPU,
the call raises.

    paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale)
    paged_attention_decode_append(out, q, new_k, new_v, k_cache, v_cache, block_tables,
                                  context_lens, scale)
    reshape_and_cache(key, value, k_cache, v_cache, slot_mapping)
    ..._fp8 variants of the three: caches are uint8 tensors of OCP FP8 E4M3 codes with
    one scale each (key = code value * k_scale, value = code value * v_scale)
    copy_blocks(caches, src_dst_pairs)
    paged_attention_decode_grouped(out, q, k_cache, v_cache, block_tables, context_lens,
                                   scale, prefix_groups(block_tables, context_lens, bs))
        the decode of a batch whose sequences share prefix blocks, each shared block
        read once per group
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, Optional, Tuple, Union

import torch

__all__ = ["paged_attention_decode", "paged_attention_decode_append", "reshape_and_cache",
           "paged_attention_decode_noalloc",
           "paged_attention_decode_fp8", "paged_attention_decode_append_fp8",
           "reshape_and_cache_fp8", "copy_blocks", "workspace_size",
           "workspace_init", "partials_layout", "version", "strerror", "PagedKVError",
           "library_path", "load", "read_tiles",
           "PreparedDecode", "PreparedReshapeAndCache", "PreparedCopyBlocks",
           "PrefixGroups", "prefix_groups", "grouped_workspace_size",
           "paged_attention_decode_grouped", "PreparedGroupedDecode"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpagedkv.so")
_lib = None

_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}

_P = ctypes.c_void_p
_I = ctypes.c_int


class PagedKVError(RuntimeError):
    """A non-zero status from the library (the message is pkv_strerror's text)."""

    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} (code {code})")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libpagedkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.pkv_version.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_strerror.restype = ctypes.c_char_p
    lib.pkv_strerror.argtypes = [_I]
    lib.pkv_paged_attention_workspace_size.restype = ctypes.c_size_t
    lib.pkv_paged_attention_workspace_size.argtypes = [_I] * 7
    lib.pkv_paged_attention_partials_layout.restype = _I
    lib.pkv_paged_attention_partials_layout.argtypes = [_I] * 8 + [_P]
    lib.pkv_workspace_init.restype = _I
    lib.pkv_workspace_init.argtypes = [_P, ctypes.c_size_t, _P]
    lib.pkv_paged_attention_decode.restype = _I
    lib.pkv_paged_attention_decode.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_float] + \
        [_I] * 9 + [_P, ctypes.c_size_t, _P]
    lib.pkv_paged_attention_decode_noalloc.restype = _I
    lib.pkv_paged_attention_decode_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_float] + \
        [_I] * 9 + [_P]
    lib.pkv_paged_attention_decode_append.restype = _I
    lib.pkv_paged_attention_decode_append.argtypes = [_P] * 8 + [ctypes.c_float] + \
        [_I] * 9 + [_P, ctypes.c_size_t, _P]
    _F = ctypes.c_float
    lib.pkv_paged_attention_decode_fp8.restype = _I
    lib.pkv_paged_attention_decode_fp8.argtypes = [_P] * 4 + [_F, _F, _P, _P, _F] + \
        [_I] * 9 + [_P, ctypes.c_size_t, _P]
    lib.pkv_paged_attention_decode_append_fp8.restype = _I
    lib.pkv_paged_attention_decode_append_fp8.argtypes = [_P] * 6 + [_F, _F, _P, _P, _F] + \
        [_I] * 9 + [_P, ctypes.c_size_t, _P]
    lib.pkv_paged_attention_chunk.restype = _I
    lib.pkv_paged_attention_chunk.argtypes = [_P] * 7 + [_F] + [_I] * 10 + [_P]
    lib.pkv_paged_attention_chunk_fp8.restype = _I
    lib.pkv_paged_attention_chunk_fp8.argtypes = [_P] * 4 + [_F, _F] + [_P] * 3 + [_F] + \
        [_I] * 10 + [_P]
    lib.pkv_reshape_and_cache_fp8.restype = _I
    lib.pkv_reshape_and_cache_fp8.argtypes = [_P] * 5 + [_F, _F] + [_I] * 6 + [_P]
    lib.pkv_reshape_and_cache.restype = _I
    lib.pkv_reshape_and_cache.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]
    lib.pkv_read_tiles.restype = _I
    lib.pkv_read_tiles.argtypes = [_P, ctypes.c_size_t, _P, _I, _I, _I, _I, _P, _P]
    lib.pkv_swap_blocks.restype = _I
    lib.pkv_swap_blocks.argtypes = [_P, _P, _P, _I, _I, _I, ctypes.c_size_t, _P]
    lib.pkv_copy_blocks.restype = _I
    lib.pkv_copy_blocks.argtypes = [_P, _P, _I, _I, ctypes.c_size_t, _P]
    lib.pkv_paged_attention_grouped_workspace_size.restype = ctypes.c_size_t
    lib.pkv_paged_attention_grouped_workspace_size.argtypes = [_I] * 3
    lib.pkv_paged_attention_decode_grouped.restype = _I
    lib.pkv_paged_attention_decode_grouped.argtypes = [_P] * 10 + [_I] * 3 + [_F] + \
        [_I] * 8 + [_P, ctypes.c_size_t, _P]
    lib.pkv_paged_attention_decode_grouped_fp8.restype = _I
    lib.pkv_paged_attention_decode_grouped_fp8.argtypes = [_P] * 6 + [_F, _F] + [_P] * 4 + \
        [_I] * 3 + [_F] + [_I] * 8 + [_P, ctypes.c_size_t, _P]
    lib.pkv_prefix_groups.restype = _I
    lib.pkv_prefix_groups.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _P, _P]
    _lib = lib
    return lib


def version() -> str:
    return load().pkv_version().decode()


def strerror(code: int) -> str:
    return load().pkv_strerror(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise PagedKVError(code, what)


def _gpu(t: torch.Tensor, name: str, dtype=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                   block_size: int, max_blocks_per_seq: int, partition_size: int = 0) -> int:
    return int(load().pkv_paged_attention_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                          head_dim, block_size,
                                                          max_blocks_per_seq, partition_size))


def partials_layout(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                    block_size: int, max_blocks_per_seq: int, partition_size: int,
                    dtype: torch.dtype) -> Tuple[int, Tuple[int, int, int]]:
    """(P, (offset of m, offset of l, offset of o)) of the per-partition records a
    decode call with this partition size leaves in its workspace (P = 0: none)."""
    offs = (ctypes.c_size_t * 3)()
    rc = load().pkv_paged_attention_partials_layout(num_seqs, num_heads, num_kv_heads,
                                                    head_dim, block_size, max_blocks_per_seq,
                                                    partition_size, _DTYPES[dtype], offs)
    if rc < 0:
        raise PagedKVError(rc, "pkv_paged_attention_partials_layout")
    return rc, (int(offs[0]), int(offs[1]), int(offs[2]))


def workspace_init(workspace: torch.Tensor) -> None:
    """Zero-fill a workspace on the current stream (needed once, before first use)."""
    _gpu(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().pkv_workspace_init(workspace.data_ptr(), nbytes, _stream(workspace.device)),
           "pkv_workspace_init")


# One zero-initialised workspace per (device, stream); the library leaves its
# bookkeeping zeroed after every call, so a workspace can be reused by later calls
# on the same stream.
_WORKSPACES: Dict[Tuple[int, int], torch.Tensor] = {}


def _workspace_for(device: torch.device, nbytes: int) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           _stream(device))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        workspace_init(ws)
        _WORKSPACES[key] = ws
    return ws


def _decode_shape(out, q, k_cache, v_cache, block_tables, context_lens, kv_fp8=False):
    """Validate the tensors of one decode call; returns (B, Hq, D, NB, Hkv, bs, MB)."""
    for name, t in (("out", out), ("q", q)):
        _gpu(t, name, q.dtype)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _gpu(t, name, torch.uint8 if kv_fp8 else q.dtype)
    _gpu(block_tables, "block_tables", torch.int32)
    _gpu(context_lens, "context_lens", torch.int32)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,Hq,D] and caches [num_blocks,Hkv,bs,D]")
    B, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    if out.shape != q.shape or D2 != D:
        raise ValueError("out must match q, and the caches' head_dim must match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    return B, Hq, D, NB, Hkv, bs, block_tables.shape[1]


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                 workspace, own_workspace, kv_fp8=False):
    """Validate one decode call; returns (ctypes argument tuple without the stream,
    the workspace tensor in use). With kv_fp8 the caches are uint8 E4M3 codes."""
    B, Hq, D, NB, Hkv, bs, MB = _decode_shape(out, q, k_cache, v_cache, block_tables,
                                              context_lens, kv_fp8)
    need = workspace_size(B, Hq, Hkv, D, bs, MB, partition_size)
    if workspace is None:
        if own_workspace and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            workspace_init(workspace)
        else:
            workspace = _workspace_for(q.device, need)
    else:
        _gpu(workspace, "workspace")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), float(scale), B, Hq, Hkv, D, bs,
            MB, NB, _DTYPES[q.dtype], int(partition_size), ws_ptr, ws_bytes)
    return args, workspace


def _new_rows(new_k, new_v, q, k_cache):
    for name, t in (("new_k", new_k), ("new_v", new_v)):
        _gpu(t, name, q.dtype)
    want = (q.shape[0], k_cache.shape[1], q.shape[2])
    if tuple(new_k.shape) != want or tuple(new_v.shape) != want:
        raise ValueError(f"new_k/new_v must be [num_seqs, num_kv_heads, head_dim] = {want}")
    return new_k.data_ptr(), new_v.data_ptr()


def _fused(args, rows):
    """Argument tuple of pkv_paged_attention_decode_append from a decode tuple."""
    return args[:2] + rows + args[2:]


def paged_attention_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                           v_cache: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, scale: float, partition_size: int = 0,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[b,h,:] = attention of q[b,h,:] over the first context_lens[b] tokens that
    block_tables[b] maps into the paged k_cache / v_cache ([num_blocks, Hkv, bs, D]).

    ``workspace``: optional uint8 device tensor, zero-filled before its first use;
    by default a cached per-(device, stream) workspace is used."""
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           partition_size, workspace, False)
    _check(load().pkv_paged_attention_decode(*args, _stream(q.device)),
           "pkv_paged_attention_decode")
    return out


def paged_attention_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, scale: float,
                                   partition_size: int = 0) -> torch.Tensor:
    """paged_attention_decode with the library's fixed scratch array instead of a
    workspace: allocates no device memory (graph capture, serving loops). Calls that
    overlap on one GPU race on that array; run them on one stream."""
    B, Hq, D, NB, Hkv, bs, MB = _decode_shape(out, q, k_cache, v_cache, block_tables,
                                              context_lens)
    _check(load().pkv_paged_attention_decode_noalloc(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), B, Hq, Hkv, D, bs, MB,
        NB, _DTYPES[q.dtype], int(partition_size), _stream(q.device)),
        "pkv_paged_attention_decode_noalloc")
    return out


def paged_attention_decode_append(out: torch.Tensor, q: torch.Tensor, new_k: torch.Tensor,
                                  new_v: torch.Tensor, k_cache: torch.Tensor,
                                  v_cache: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, scale: float,
                                  partition_size: int = 0,
                                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step: new_k[b]/new_v[b] ([B, Hkv, D]) are written at position
    context_lens[b] - 1 of sequence b (the slot its block table gives), then q attends
    over all context_lens[b] tokens. On the matrix-core paths this is one kernel."""
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           partition_size, workspace, False)
    rows = _new_rows(new_k, new_v, q, k_cache)
    _check(load().pkv_paged_attention_decode_append(*_fused(args, rows), _stream(q.device)),
           "pkv_paged_attention_decode_append")
    return out


def _with_scales(args, at, k_scale, v_scale):
    """Insert the two cache scales into a ctypes argument tuple at position `at`."""
    if not (float(k_scale) > 0 and float(v_scale) > 0):
        raise ValueError("cache scales must be positive")
    return args[:at] + (float(k_scale), float(v_scale)) + args[at:]


def paged_attention_decode_fp8(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                               v_cache: torch.Tensor, k_scale: float, v_scale: float,
                               block_tables: torch.Tensor, context_lens: torch.Tensor,
                               scale: float, partition_size: int = 0,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """paged_attention_decode over 8-bit caches: k_cache/v_cache are uint8 tensors of
    OCP FP8 E4M3 codes [num_blocks, Hkv, bs, D]; key = code value * k_scale, value =
    code value * v_scale. q/out are bfloat16 or float16."""
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           partition_size, workspace, False, kv_fp8=True)
    _check(load().pkv_paged_attention_decode_fp8(*_with_scales(args, 4, k_scale, v_scale),
                                                 _stream(q.device)),
           "pkv_paged_attention_decode_fp8")
    return out


def paged_attention_decode_append_fp8(out, q, new_k, new_v, k_cache, v_cache, k_scale,
                                      v_scale, block_tables, context_lens, scale,
                                      partition_size: int = 0,
                                      workspace: Optional[torch.Tensor] = None):
    """paged_attention_decode_append over 8-bit caches: new_k/new_v (q's dtype) are
    quantised (float32(x) * float32(1/scale), nearest E4M3, saturating at 448) into
    each sequence's context-end slot, then attended."""
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           partition_size, workspace, False, kv_fp8=True)
    fused = _fused(args, _new_rows(new_k, new_v, q, k_cache))
    _check(load().pkv_paged_attention_decode_append_fp8(
        *_with_scales(fused, 6, k_scale, v_scale), _stream(q.device)),
        "pkv_paged_attention_decode_append_fp8")
    return out


def _chunk_args(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                max_query_len, kv_fp8):
    for name, t in (("out", out), ("q", q)):
        _gpu(t, name, q.dtype)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _gpu(t, name, torch.uint8 if kv_fp8 else q.dtype)
    for name, t in (("block_tables", block_tables), ("context_lens", context_lens),
                    ("query_start", query_start)):
        _gpu(t, name, torch.int32)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.dim() != 3 or out.shape != q.shape or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape or k_cache.shape[3] != q.shape[2]:
        raise ValueError("expected q/out [num_query_tokens,Hq,D] and caches "
                         "[num_blocks,Hkv,bs,D] with the same D")
    B = context_lens.shape[0]
    if context_lens.dim() != 1 or query_start.shape != (B + 1,) or block_tables.dim() != 2 \
            or block_tables.shape[0] != B:
        raise ValueError("context_lens [B], query_start [B + 1], block_tables [B, max_blocks]")
    if max_query_len is None:
        max_query_len = int((query_start[1:] - query_start[:-1]).max()) if B else 0
    NQ, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    return (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(),
            float(scale), B, NQ, int(max_query_len), Hq, Hkv, D, bs, block_tables.shape[1], NB,
            _DTYPES[q.dtype])


def paged_attention_chunk(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, block_tables: torch.Tensor,
                          context_lens: torch.Tensor, query_start: torch.Tensor, scale: float,
                          max_query_len: Optional[int] = None, k_scale: Optional[float] = None,
                          v_scale: Optional[float] = None) -> torch.Tensor:
    """Attention of several new query tokens per sequence (causal within the chunk).

    q/out [num_query_tokens, Hq, D]; sequence b owns rows query_start[b] ..
    query_start[b+1]-1, its last T_b context tokens (their K/V already in the cache);
    row j attends the first context_lens[b] - T_b + j + 1 tokens. ``max_query_len``
    (>= every T_b) is read from query_start when not given (a device sync).
    With uint8 caches (E4M3 codes) pass k_scale and v_scale."""
    fp8 = k_cache.dtype == torch.uint8
    args = _chunk_args(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                       scale, max_query_len, fp8)
    if fp8:
        if k_scale is None or v_scale is None:
            raise ValueError("8-bit caches need k_scale and v_scale")
        _check(load().pkv_paged_attention_chunk_fp8(*_with_scales(args, 4, k_scale, v_scale),
                                                    _stream(q.device)),
               "pkv_paged_attention_chunk_fp8")
    else:
        _check(load().pkv_paged_attention_chunk(*args, _stream(q.device)),
               "pkv_paged_attention_chunk")
    return out


class PreparedChunk:
    """paged_attention_chunk validated once for a fixed set of tensors (serving loops,
    HIP graph capture); calling it enqueues the kernel on ``stream`` or the current
    stream of the tensors' device."""

    def __init__(self, out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                 scale, max_query_len: int, k_scale: Optional[float] = None,
                 v_scale: Optional[float] = None):
        fp8 = k_cache.dtype == torch.uint8
        self._args = _chunk_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                 query_start, scale, max_query_len, fp8)
        self._name = "pkv_paged_attention_chunk"
        if fp8:
            if k_scale is None or v_scale is None:
                raise ValueError("8-bit caches need k_scale and v_scale")
            self._args = _with_scales(self._args, 4, k_scale, v_scale)
            self._name += "_fp8"
        self._fn = getattr(load(), self._name)
        self._device = q.device
        self.out = out
        self._keep = (out, q, k_cache, v_cache, block_tables, context_lens, query_start)

    def __call__(self, stream: Optional[int] = None) -> torch.Tensor:
        st = _stream(self._device) if stream is None else stream
        rc = self._fn(*self._args, st)
        if rc != 0:
            raise PagedKVError(rc, self._name)
        return self.out


class PreparedDecode:
    """A decode call validated once for a fixed set of tensors, for loops that run
    it many times (serving steps, HIP graph capture). It owns a zero-initialised
    workspace unless one is passed. Calling it enqueues the decode on ``stream`` (a
    raw hipStream_t handle) or on the current stream of the tensors' device. With
    ``new_k``/``new_v`` it is the fused step of paged_attention_decode_append."""

    def __init__(self, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                 partition_size: int = 0, workspace: Optional[torch.Tensor] = None,
                 new_k: Optional[torch.Tensor] = None, new_v: Optional[torch.Tensor] = None,
                 k_scale: Optional[float] = None, v_scale: Optional[float] = None):
        fp8 = k_cache.dtype == torch.uint8
        if fp8 and (k_scale is None or v_scale is None):
            raise ValueError("8-bit caches need k_scale and v_scale")
        self._args, self.workspace = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                  context_lens, scale, partition_size,
                                                  workspace, True, kv_fp8=fp8)
        if (new_k is None) != (new_v is None):
            raise ValueError("pass both new_k and new_v, or neither")
        if new_k is not None:
            self._args = _fused(self._args, _new_rows(new_k, new_v, q, k_cache))
            self._name = "pkv_paged_attention_decode_append"
            at = 6
        else:
            self._name = "pkv_paged_attention_decode"
            at = 4
        if fp8:
            self._args = _with_scales(self._args, at, k_scale, v_scale)
            self._name += "_fp8"
        self._fn = getattr(load(), self._name)
        self._device = q.device
        self.out = out
        # the raw pointers above stay valid only while these tensors are alive
        self._keep = (out, q, k_cache, v_cache, block_tables, context_lens, new_k, new_v)

    def __call__(self, stream: Optional[int] = None) -> torch.Tensor:
        st = _stream(self._device) if stream is None else stream
        rc = self._fn(*self._args, st)
        if rc != 0:
            raise PagedKVError(rc, self._name)
        return self.out


class PrefixGroups:
    """Groups of consecutive sequences sharing prefix blocks (see prefix_groups):
    group_start [num_groups + 1] and group_prefix [num_groups] as int32 tensors on the
    batch's device, and the bounds the grouped decode is sized by."""

    def __init__(self, group_start: torch.Tensor, group_prefix: torch.Tensor,
                 max_group_size: int, max_prefix_blocks: int):
        self.group_start = group_start
        self.group_prefix = group_prefix
        self.num_groups = int(group_prefix.shape[0])
        self.max_group_size = int(max_group_size)
        self.max_prefix_blocks = int(max_prefix_blocks)


def prefix_groups(block_tables: torch.Tensor, context_lens: torch.Tensor,
                  block_size: int, device: Optional[torch.device] = None) -> PrefixGroups:
    """Host derivation of the groups (pkv_prefix_groups): maximal runs of sequences
    whose first table entry is the same block, with the leading entries they share as
    full blocks. Reads host copies of the tables (a device sync when they are on the
    GPU); the groups are placed on ``device`` (default: the tables' device)."""
    if block_tables.dim() != 2 or context_lens.dim() != 1 or \
            context_lens.shape[0] != block_tables.shape[0]:
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    dev = block_tables.device if device is None else torch.device(device)
    t = block_tables.detach().to("cpu", torch.int32).contiguous()
    c = context_lens.detach().to("cpu", torch.int32).contiguous()
    B, MB = t.shape
    start = torch.empty(B + 1, dtype=torch.int32)
    pfx = torch.empty(max(B, 1), dtype=torch.int32)
    ng, gmax, pmax = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(load().pkv_prefix_groups(t.data_ptr(), c.data_ptr(), B, MB, int(block_size),
                                    start.data_ptr(), pfx.data_ptr(), ctypes.byref(ng),
                                    ctypes.byref(gmax), ctypes.byref(pmax)),
           "pkv_prefix_groups")
    n = ng.value
    return PrefixGroups(start[:n + 1].to(dev), pfx[:n].to(dev), gmax.value, pmax.value)


def grouped_workspace_size(num_seqs: int, num_heads: int, max_prefix_blocks: int) -> int:
    return int(load().pkv_paged_attention_grouped_workspace_size(num_seqs, num_heads,
                                                                  max_prefix_blocks))


class PreparedGroupedDecode:
    """The grouped decode (pkv_paged_attention_decode_grouped) validated once for a
    fixed set of tensors: prefix blocks shared by a group's sequences are read once for
    the group's tile of members. With ``new_k``/``new_v`` it is the fused step (append,
    then attend); uint8 caches (E4M3 codes) need k_scale and v_scale. It owns a
    workspace (needed only for prefixes of more than 128 blocks) unless one is
    passed."""

    def __init__(self, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                 groups: PrefixGroups, new_k: Optional[torch.Tensor] = None,
                 new_v: Optional[torch.Tensor] = None, k_scale: Optional[float] = None,
                 v_scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None):
        fp8 = k_cache.dtype == torch.uint8
        if fp8 and (k_scale is None or v_scale is None):
            raise ValueError("8-bit caches need k_scale and v_scale")
        B, Hq, D, NB, Hkv, bs, MB = _decode_shape(out, q, k_cache, v_cache, block_tables,
                                                  context_lens, fp8)
        _gpu(groups.group_start, "group_start", torch.int32)
        _gpu(groups.group_prefix, "group_prefix", torch.int32)
        if groups.group_start.shape != (groups.num_groups + 1,):
            raise ValueError("group_start must hold num_groups + 1 entries")
        if (new_k is None) != (new_v is None):
            raise ValueError("pass both new_k and new_v, or neither")
        rows = _new_rows(new_k, new_v, q, k_cache) if new_k is not None else (None, None)
        need = grouped_workspace_size(B, Hq, groups.max_prefix_blocks)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif workspace is not None:
            _gpu(workspace, "workspace")
        self.workspace = workspace
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() if workspace is not None else 0
        head = (out.data_ptr(), q.data_ptr()) + rows + (k_cache.data_ptr(),
                                                        v_cache.data_ptr())
        tail = (block_tables.data_ptr(), context_lens.data_ptr(),
                groups.group_start.data_ptr(), groups.group_prefix.data_ptr(),
                groups.num_groups, groups.max_group_size, groups.max_prefix_blocks,
                float(scale), B, Hq, Hkv, D, bs, MB, NB, _DTYPES[q.dtype], ws_ptr, ws_bytes)
        self._name = "pkv_paged_attention_decode_grouped"
        if fp8:
            if not (float(k_scale) > 0 and float(v_scale) > 0):
                raise ValueError("cache scales must be positive")
            self._args = head + (float(k_scale), float(v_scale)) + tail
            self._name += "_fp8"
        else:
            self._args = head + tail
        self._fn = getattr(load(), self._name)
        self._device = q.device
        self.out = out
        self._keep = (out, q, k_cache, v_cache, block_tables, context_lens, new_k, new_v,
                      groups.group_start, groups.group_prefix)

    def __call__(self, stream: Optional[int] = None) -> torch.Tensor:
        st = _stream(self._device) if stream is None else stream
        rc = self._fn(*self._args, st)
        if rc != 0:
            raise PagedKVError(rc, self._name)
        return self.out


def paged_attention_decode_grouped(out, q, k_cache, v_cache, block_tables, context_lens,
                                   scale, groups: PrefixGroups, new_k=None, new_v=None,
                                   k_scale=None, v_scale=None,
                                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """paged_attention_decode (or, with new_k/new_v, paged_attention_decode_append) for
    a batch whose groups of sequences share prefix blocks: each shared block is read
    once per group. ``groups`` comes from prefix_groups or is built by the caller."""
    return PreparedGroupedDecode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                 groups, new_k, new_v, k_scale, v_scale, workspace)()


def _append_args(key, value, k_cache, v_cache, slot_mapping):
    for name, t in (("key", key), ("value", value), ("k_cache", k_cache), ("v_cache", v_cache)):
        _gpu(t, name, key.dtype)
    _gpu(slot_mapping, "slot_mapping", torch.int64)
    if key.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {key.dtype}")
    if key.dim() != 3 or value.shape != key.shape or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape:
        raise ValueError("expected key/value [T,Hkv,D] and caches [num_blocks,Hkv,bs,D]")
    T, Hkv, D = key.shape
    NB, Hkv2, bs, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or slot_mapping.shape != (T,):
        raise ValueError("key/value and caches disagree on heads/head_dim, or slot_mapping != [T]")
    return (key.data_ptr(), value.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            slot_mapping.data_ptr(), T, Hkv, D, bs, NB, _DTYPES[key.dtype])


def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float,
                          v_scale: float) -> None:
    """Quantising slot-mapped append into 8-bit caches (uint8 E4M3 codes): key/value
    ([T, Hkv, D], float32/bfloat16/float16) at slot_mapping[t]."""
    for name, t in (("key", key), ("value", value)):
        _gpu(t, name, key.dtype)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _gpu(t, name, torch.uint8)
    _gpu(slot_mapping, "slot_mapping", torch.int64)
    if key.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {key.dtype}")
    if key.dim() != 3 or value.shape != key.shape or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape:
        raise ValueError("expected key/value [T,Hkv,D] and caches [num_blocks,Hkv,bs,D]")
    T, Hkv, D = key.shape
    NB, Hkv2, bs, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or slot_mapping.shape != (T,):
        raise ValueError("key/value and caches disagree on heads/head_dim, or slot_mapping != [T]")
    args = (key.data_ptr(), value.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            slot_mapping.data_ptr(), float(k_scale), float(v_scale), T, Hkv, D, bs, NB,
            _DTYPES[key.dtype])
    _check(load().pkv_reshape_and_cache_fp8(*args, _stream(key.device)),
           "pkv_reshape_and_cache_fp8")


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Write key[t]/value[t] ([T, Hkv, D]) into the caches at slot_mapping[t]
    (int64, physical_block * block_size + offset; negative = skip)."""
    args = _append_args(key, value, k_cache, v_cache, slot_mapping)
    _check(load().pkv_reshape_and_cache(*args, _stream(key.device)), "pkv_reshape_and_cache")


class PreparedReshapeAndCache:
    """reshape_and_cache validated once for a fixed set of tensors (see PreparedDecode)."""

    def __init__(self, key, value, k_cache, v_cache, slot_mapping):
        self._args = _append_args(key, value, k_cache, v_cache, slot_mapping)
        self._fn = load().pkv_reshape_and_cache
        self._device = key.device
        self._keep = (key, value, k_cache, v_cache, slot_mapping)

    def __call__(self, stream: Optional[int] = None) -> None:
        st = _stream(self._device) if stream is None else stream
        rc = self._fn(*self._args, st)
        if rc != 0:
            raise PagedKVError(rc, "pkv_reshape_and_cache")


def _copy_args(caches, src_dst_pairs):
    if isinstance(caches, torch.Tensor):
        caches = [caches]
    _gpu(src_dst_pairs, "src_dst_pairs", torch.int32)
    if src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be [n, 2]")
    n = src_dst_pairs.shape[0]
    args = []
    for c in caches:
        _gpu(c, "cache")
        nb = c.shape[0]
        block_bytes = (c.numel() // nb) * c.element_size() if nb else 0
        args.append((c.data_ptr(), src_dst_pairs.data_ptr(), n, nb, block_bytes))
    return list(caches), args


def copy_blocks(caches: Union[torch.Tensor, Iterable[torch.Tensor]],
                src_dst_pairs: torch.Tensor) -> None:
    """For each (src, dst) row of src_dst_pairs (int32 [n, 2] on the device), copy
    block src to block dst in every pool of ``caches``."""
    caches, args = _copy_args(caches, src_dst_pairs)
    for c, a in zip(caches, args):
        _check(load().pkv_copy_blocks(*a, _stream(c.device)), "pkv_copy_blocks")


class PreparedCopyBlocks:
    """copy_blocks validated once for fixed pools and pairs (see PreparedDecode)."""

    def __init__(self, caches, src_dst_pairs):
        caches, self._args = _copy_args(caches, src_dst_pairs)
        self._fn = load().pkv_copy_blocks
        self._device = src_dst_pairs.device
        self._keep = (caches, src_dst_pairs)

    def __call__(self, stream: Optional[int] = None) -> None:
        st = _stream(self._device) if stream is None else stream
        for a in self._args:
            rc = self._fn(*a, st)
            if rc != 0:
                raise PagedKVError(rc, "pkv_copy_blocks")


def _swap_args(dst_pool, src_pool, src_dst_pairs):
    pools = (("dst_pool", dst_pool), ("src_pool", src_pool))
    dev = [t.device for _, t in pools if t.is_cuda]
    if not dev:
        raise ValueError("at least one pool must be on the GPU")
    for name, t in pools:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not t.is_cuda and not t.is_pinned():
            raise ValueError(f"{name} is host memory that is not pinned (use pin_memory=True)")
        if t.is_cuda and t.device != dev[0]:
            raise ValueError("device pools must be on one device")
    if dst_pool.dtype != src_pool.dtype or dst_pool.shape[1:] != src_pool.shape[1:]:
        raise ValueError("pools must share dtype and block layout [blocks, ...]")
    if src_dst_pairs.dtype != torch.int32 or not src_dst_pairs.is_contiguous():
        raise ValueError("src_dst_pairs must be a contiguous int32 tensor")
    if src_dst_pairs.is_cuda:
        if src_dst_pairs.device != dev[0]:
            raise ValueError("src_dst_pairs must be on the pools' device")
    elif not src_dst_pairs.is_pinned():
        raise ValueError("src_dst_pairs must be on the GPU or in pinned host memory")
    p = src_dst_pairs.reshape(-1, 2)
    bb = dst_pool[0].numel() * dst_pool.element_size() if dst_pool.shape[0] else \
        int(torch.tensor(dst_pool.shape[1:]).prod()) * dst_pool.element_size()
    return (dst_pool.data_ptr(), src_pool.data_ptr(), p.data_ptr(), p.shape[0],
            src_pool.shape[0], dst_pool.shape[0], bb), dev[0]


def swap_blocks(dst_pool: torch.Tensor, src_pool: torch.Tensor,
                src_dst_pairs: torch.Tensor) -> None:
    """Copy block src of src_pool over block dst of dst_pool for each (src, dst) pair
    (int32 [n, 2] on the GPU or in pinned host memory). One pool is a GPU tensor, the other a GPU tensor or a
    pinned CPU tensor (pin_memory=True) of the same dtype and block layout: swap-out
    passes the host pool as dst_pool, swap-in as src_pool. Enqueued on the GPU's
    current stream; host memory is complete once that stream is synchronised."""
    args, dev = _swap_args(dst_pool, src_pool, src_dst_pairs)
    _check(load().pkv_swap_blocks(*args, _stream(dev)), "pkv_swap_blocks")


class PreparedSwapBlocks:
    """swap_blocks validated once for a fixed set of tensors."""

    def __init__(self, dst_pool, src_pool, src_dst_pairs):
        self._args, self._device = _swap_args(dst_pool, src_pool, src_dst_pairs)
        self._fn = load().pkv_swap_blocks
        self._keep = (dst_pool, src_pool, src_dst_pairs)

    def __call__(self, stream: Optional[int] = None) -> None:
        st = _stream(self._device) if stream is None else stream
        rc = self._fn(*self._args, st)
        if rc != 0:
            raise PagedKVError(rc, "pkv_swap_blocks")


def read_tiles(base: torch.Tensor, offsets: torch.Tensor, tile_bytes: int, workgroups: int,
               tiles_in_flight: int, sink: torch.Tensor) -> None:
    """Bandwidth probe (diagnostic): read the tiles of tile_bytes bytes at byte offsets
    ``offsets`` (int64, on the GPU) of the GPU tensor ``base``; ``sink`` is an int32 GPU
    tensor of at least workgroups * 256 elements."""
    _gpu(base, "base")
    _gpu(offsets, "offsets", torch.int64)
    _gpu(sink, "sink", torch.int32)
    if sink.numel() < workgroups * 256:
        raise ValueError("sink needs workgroups * 256 elements")
    _check(load().pkv_read_tiles(base.data_ptr(), base.numel() * base.element_size(),
                                 offsets.data_ptr(), offsets.numel(), tile_bytes, workgroups,
                                 tiles_in_flight, sink.data_ptr(), _stream(base.device)),
           "pkv_read_tiles")
