"""Python binding of the host block manager (include/pagedattn_blocks.h):
argument marshalling only; the allocator, its reference counts and
copy-on-write live in the library (csrc/pa_blocks.cpp)."""
from __future__ import annotations

import ctypes

import numpy as np

from . import PA_OK, PagedAttentionError, _check, _ptr, _stream, load_library

PA_ENOMEM = -5

_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)


class BmStats(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("free_blocks", ctypes.c_int32),
        ("used_blocks", ctypes.c_int32),
        ("shared_blocks", ctypes.c_int32),
        ("num_sequences", ctypes.c_int32),
        ("pad", ctypes.c_int32),
        ("logical_tokens", ctypes.c_int64),
        ("stored_tokens", ctypes.c_int64),
        ("utilization", ctypes.c_double),
    ]


_configured = False


def _lib():
    global _configured
    lib = load_library()
    if not _configured:
        P, I, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.pa_bm_create.restype = P
        lib.pa_bm_create.argtypes = [I, I]
        lib.pa_bm_destroy.restype = None
        lib.pa_bm_destroy.argtypes = [P]
        lib.pa_bm_add.restype = ctypes.c_int
        lib.pa_bm_add.argtypes = [P, I64, I, _I32P]
        lib.pa_bm_add_shared.restype = ctypes.c_int
        lib.pa_bm_add_shared.argtypes = [P, I64, I64, I, I, _I32P]
        lib.pa_bm_fork.restype = ctypes.c_int
        lib.pa_bm_fork.argtypes = [P, I64, I64]
        lib.pa_bm_append.restype = ctypes.c_int
        lib.pa_bm_append.argtypes = [P, I64, I, _I32P, _I32P, _I32P]
        lib.pa_bm_free.restype = ctypes.c_int
        lib.pa_bm_free.argtypes = [P, I64]
        lib.pa_bm_length.restype = I
        lib.pa_bm_length.argtypes = [P, I64]
        lib.pa_bm_tables.restype = ctypes.c_int
        lib.pa_bm_tables.argtypes = [P, _I64P, I, _I32P, I, _I32P]
        lib.pa_bm_prefix_groups.restype = ctypes.c_int
        lib.pa_bm_prefix_groups.argtypes = [P, _I64P, I, _I32P, _I32P, _I32P, _I32P, _I32P]
        lib.pa_bm_get_stats.restype = ctypes.c_int
        lib.pa_bm_get_stats.argtypes = [P, ctypes.POINTER(BmStats)]
        lib.pa_bm_refcount.restype = I
        lib.pa_bm_refcount.argtypes = [P, I]
        lib.pa_validate_batch.restype = ctypes.c_int
        lib.pa_validate_batch.argtypes = [I, I, _I32P, _I32P, _I32P, _I32P, I, I, _I32P, _I32P]
        lib.pa_copy_blocks.restype = ctypes.c_int
        lib.pa_copy_blocks.argtypes = [ctypes.c_void_p, P, P, P, P, P, ctypes.c_int, P]
        _configured = True
    return lib


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _p32(a):
    return None if a is None else a.ctypes.data_as(_I32P)


class BlockManager:
    """Physical-block allocator of one paged cache: free list, block tables,
    reference counts with copy-on-write, slot mapping."""

    def __init__(self, num_blocks: int, max_blocks_per_seq: int):
        self._lib = _lib()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(max_blocks_per_seq))
        if not self._h:
            raise PagedAttentionError("pa_bm_create failed")
        self.num_blocks = int(num_blocks)
        self.max_blocks_per_seq = int(max_blocks_per_seq)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def add(self, seq: int, num_tokens: int) -> np.ndarray:
        """New sequence of num_tokens tokens; returns their slots."""
        slots = np.empty(max(num_tokens, 1), np.int32)
        _check(self._lib.pa_bm_add(self._h, seq, num_tokens, _p32(slots)), "pa_bm_add")
        return slots[:num_tokens]

    def add_shared(self, seq: int, owner: int, prefix_blocks: int, num_tokens: int) -> np.ndarray:
        """New sequence sharing owner's first prefix_blocks (full) blocks,
        then num_tokens tokens of its own; returns the slots of those."""
        slots = np.empty(max(num_tokens, 1), np.int32)
        _check(self._lib.pa_bm_add_shared(self._h, seq, owner, prefix_blocks, num_tokens,
                                          _p32(slots)), "pa_bm_add_shared")
        return slots[:num_tokens]

    def fork(self, parent: int, child: int) -> None:
        _check(self._lib.pa_bm_fork(self._h, parent, child), "pa_bm_fork")

    def append(self, seq: int, num_tokens: int = 1):
        """Returns (slots, copies): copies is a list of (src, dst) block
        pairs the cache must copy before the new rows are written."""
        slots = np.empty(max(num_tokens, 1), np.int32)
        pair = np.empty(2, np.int32)
        n = np.zeros(1, np.int32)
        _check(self._lib.pa_bm_append(self._h, seq, num_tokens, _p32(slots), _p32(pair),
                                      _p32(n)), "pa_bm_append")
        return slots[:num_tokens], [(int(pair[0]), int(pair[1]))] if n[0] else []

    def free(self, seq: int) -> None:
        _check(self._lib.pa_bm_free(self._h, seq), "pa_bm_free")

    def length(self, seq: int) -> int:
        return int(self._lib.pa_bm_length(self._h, seq))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_refcount(self._h, block))

    def tables(self, seqs, row_stride: int | None = None):
        """(block_tables [n][row_stride] int32, context_lens [n] int32)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = len(seqs)
        stride = self.max_blocks_per_seq if row_stride is None else int(row_stride)
        tab = np.empty((max(n, 1), stride), np.int32)
        lens = np.empty(max(n, 1), np.int32)
        _check(self._lib.pa_bm_tables(self._h, seqs.ctypes.data_as(_I64P), n, _p32(tab), stride,
                                      _p32(lens)), "pa_bm_tables")
        return tab[:n], lens[:n]

    def prefix_groups(self, seqs):
        """(groups as lists of batch indices, shared prefix blocks per group)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = len(seqs)
        off = np.empty(n + 1, np.int32)
        mem = np.empty(max(n, 1), np.int32)
        pb = np.empty(max(n, 1), np.int32)
        ng = np.zeros(1, np.int32)
        nm = np.zeros(1, np.int32)
        _check(self._lib.pa_bm_prefix_groups(self._h, seqs.ctypes.data_as(_I64P), n, _p32(off),
                                             _p32(mem), _p32(pb), _p32(ng), _p32(nm)),
               "pa_bm_prefix_groups")
        groups = [mem[off[g]:off[g + 1]].tolist() for g in range(int(ng[0]))]
        return groups, pb[:int(ng[0])].tolist()

    def stats(self) -> BmStats:
        st = BmStats()
        _check(self._lib.pa_bm_get_stats(self._h, ctypes.byref(st)), "pa_bm_get_stats")
        return st


def validate_batch(num_blocks, max_blocks_per_seq, block_tables, context_lens,
                   query_start_loc=None, slot_mapping=None, refcounts=None):
    """Host check of a batch's metadata; returns (ok, offending index)."""
    bt = _i32(block_tables)
    cl = _i32(context_lens)
    qsl = _i32(query_start_loc)
    sm = _i32(slot_mapping)
    rc = _i32(refcounts)
    S = len(cl)
    T = int(qsl[-1]) if qsl is not None else S
    bad = np.zeros(1, np.int32)
    r = _lib().pa_validate_batch(int(num_blocks), int(max_blocks_per_seq), _p32(bt), _p32(cl),
                                 _p32(qsl), _p32(sm), S, T, _p32(rc), _p32(bad))
    return r == PA_OK, int(bad[0])


def copy_blocks(shape, k_cache, v_cache, pairs, *, k_scale=None, v_scale=None, stream=None):
    """Device: copy blocks pairs[k][0] -> pairs[k][1] of both caches (and the
    fp8 scales); pairs is a device int32 tensor [n][2]."""
    n = int(pairs.shape[0]) if pairs is not None else 0
    _check(_lib().pa_copy_blocks(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                 _ptr(v_scale), _ptr(pairs), n, _stream(stream)),
           "pa_copy_blocks")
