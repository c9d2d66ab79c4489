"""Python view of the library's host block manager (pkv_bm_* in include/pagedkv.h).

Argument marshalling only; the decisions (free list, reference counts,
copy-on-write, prefix cache, eviction) are made by the C++ code in
csrc/block_manager.cpp.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import PagedKVError, load

PKV_E_NOSPACE = -9

_P, _I, _L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
_bound = False


class NoSpace(PagedKVError):
    """No free or evictable block is left for the request (nothing was changed)."""


def _lib():
    global _bound
    lib = load()
    if not _bound:
        lib.pkv_bm_create.restype = _P
        lib.pkv_bm_create.argtypes = [_I, _I, _P]
        lib.pkv_bm_destroy.restype = None
        lib.pkv_bm_destroy.argtypes = [_P]
        lib.pkv_bm_available.restype = _I
        lib.pkv_bm_available.argtypes = [_P]
        lib.pkv_bm_can_allocate.restype = _I
        lib.pkv_bm_can_allocate.argtypes = [_P, _I]
        lib.pkv_bm_add_sequence.restype = _I
        lib.pkv_bm_add_sequence.argtypes = [_P, _L, _I, _P, _P]
        lib.pkv_bm_fork.restype = _I
        lib.pkv_bm_fork.argtypes = [_P, _L, _L]
        lib.pkv_bm_append_token.restype = _I
        lib.pkv_bm_append_token.argtypes = [_P, _L, ctypes.c_int32, _P, _P, _P]
        lib.pkv_bm_append_tokens.restype = _I
        lib.pkv_bm_append_tokens.argtypes = [_P, _P, _P, _I, _P, _P]
        lib.pkv_bm_free_sequence.restype = _I
        lib.pkv_bm_free_sequence.argtypes = [_P, _L]
        lib.pkv_bm_num_tokens.restype = _L
        lib.pkv_bm_num_tokens.argtypes = [_P, _L]
        lib.pkv_bm_block_table.restype = _I
        lib.pkv_bm_block_table.argtypes = [_P, _L, _P, _I]
        lib.pkv_bm_refcount.restype = _I
        lib.pkv_bm_refcount.argtypes = [_P, ctypes.c_int32]
        lib.pkv_bm_build_tables.restype = _I
        lib.pkv_bm_build_tables.argtypes = [_P, _P, _I, _I, _P, _P]
        _bound = True
    return lib


def _check(rc: int, what: str) -> int:
    if rc == PKV_E_NOSPACE:
        raise NoSpace(rc, what)
    if rc < 0:
        raise PagedKVError(rc, what)
    return rc


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class BlockManager:
    """Block placement of a paged KV cache over ``num_blocks`` blocks of
    ``block_size`` tokens; ``order`` is the hand-out order of the free list."""

    def __init__(self, num_blocks: int, block_size: int, order: Optional[Sequence[int]] = None):
        self._l = _lib()
        self.bs = block_size
        self.num_blocks = num_blocks
        o = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
        h = self._l.pkv_bm_create(num_blocks, block_size, None if o is None else _ptr(o))
        if not h:
            raise ValueError("pkv_bm_create rejected its arguments")
        self._h = ctypes.c_void_p(h)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._l.pkv_bm_destroy(h)
            self._h = None

    def available(self) -> int:
        return _check(self._l.pkv_bm_available(self._h), "pkv_bm_available")

    def can_allocate(self, num_tokens: int) -> bool:
        return bool(_check(self._l.pkv_bm_can_allocate(self._h, num_tokens),
                           "pkv_bm_can_allocate"))

    def add_sequence(self, sid: int, num_tokens: int,
                     token_ids: Optional[Sequence[int]] = None) -> int:
        ids = None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int32)
        if ids is not None and ids.size != num_tokens:
            raise ValueError("one token id per prompt token")
        got = ctypes.c_int(0)
        _check(self._l.pkv_bm_add_sequence(self._h, sid, num_tokens,
                                           None if ids is None else _ptr(ids),
                                           ctypes.byref(got)), "pkv_bm_add_sequence")
        return got.value

    def fork(self, parent: int, child: int) -> None:
        _check(self._l.pkv_bm_fork(self._h, parent, child), "pkv_bm_fork")

    def append_token(self, sid: int, token_id: int = 0) -> Tuple[int, Optional[Tuple[int, int]]]:
        slot, src, dst = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
        _check(self._l.pkv_bm_append_token(self._h, sid, token_id, ctypes.byref(slot),
                                           ctypes.byref(src), ctypes.byref(dst)),
               "pkv_bm_append_token")
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_tokens(self, sids: Sequence[int], token_ids: Optional[Sequence[int]] = None):
        """One decode step for a batch: (count placed, slots int64 [n], copy pairs
        int32 [n, 2] with -1 where no copy is needed)."""
        s = np.ascontiguousarray(sids, dtype=np.int64)
        t = None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int32)
        slots = np.full(s.size, -1, dtype=np.int64)
        pairs = np.full((s.size, 2), -1, dtype=np.int32)
        n = _check(self._l.pkv_bm_append_tokens(self._h, _ptr(s), None if t is None else _ptr(t),
                                                s.size, _ptr(slots), _ptr(pairs)),
                   "pkv_bm_append_tokens")
        return n, slots, pairs

    def free_sequence(self, sid: int) -> None:
        _check(self._l.pkv_bm_free_sequence(self._h, sid), "pkv_bm_free_sequence")

    def num_tokens(self, sid: int) -> int:
        return _check(self._l.pkv_bm_num_tokens(self._h, sid), "pkv_bm_num_tokens")

    def block_table(self, sid: int) -> List[int]:
        n = _check(self._l.pkv_bm_block_table(self._h, sid, None, 0), "pkv_bm_block_table")
        out = np.empty(n, dtype=np.int32)
        _check(self._l.pkv_bm_block_table(self._h, sid, _ptr(out), n), "pkv_bm_block_table")
        return out.tolist()

    def refcount(self, block: int) -> int:
        return _check(self._l.pkv_bm_refcount(self._h, block), "pkv_bm_refcount")

    def build_tables(self, sids: Sequence[int], width: int):
        """(int32 [n, width] tables padded with -1, int32 [n] context lengths)."""
        s = np.ascontiguousarray(sids, dtype=np.int64)
        tables = np.empty((s.size, width), dtype=np.int32)
        lens = np.empty(s.size, dtype=np.int32)
        _check(self._l.pkv_bm_build_tables(self._h, _ptr(s), s.size, width, _ptr(tables),
                                           _ptr(lens)), "pkv_bm_build_tables")
        return tables, lens
