"""Python binding of the host block manager of libpagedkv.so
(include/pkv_block_manager.h): block pool, per-sequence block tables and
prefix cache.  Argument marshalling only; the manager is C++.

    bm = BlockManager(num_blocks, block_size)
    cached = bm.add(seq_id, prompt_tokens)     # KV of tokens[cached:] to compute
    bm.append(seq_id, new_tokens)
    bm.fork(parent, child); bm.release(seq_id)
    copies = bm.take_copies()                  # [(src, dst, valid_tokens)]
    tables, lens = bm.export(seq_ids, width)   # numpy int32, kernel inputs
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import PKV_OK, PagedKVError, lib

PKV_ENOSPACE = -4


class NoSpace(PagedKVError):
    """Not enough free or evictable blocks; the manager is unchanged."""


_P, _I32, _I64 = C.c_void_p, C.c_int32, C.c_int64


def _setup(L):
    L.pkv_bm_create.restype = _P
    L.pkv_bm_create.argtypes = [_I32, _I32, _I64]
    L.pkv_bm_destroy.restype = None
    L.pkv_bm_destroy.argtypes = [_P]
    L.pkv_bm_add.restype = C.c_int
    L.pkv_bm_add.argtypes = [_P, _I64, _P, _I32, _P]
    L.pkv_bm_append.restype = C.c_int
    L.pkv_bm_append.argtypes = [_P, _I64, _P, _I32]
    L.pkv_bm_append_batch.restype = _I32
    L.pkv_bm_append_batch.argtypes = [_P, _P, _I32, _P, _P]
    L.pkv_bm_fork.restype = C.c_int
    L.pkv_bm_fork.argtypes = [_P, _I64, _I64]
    L.pkv_bm_release.restype = C.c_int
    L.pkv_bm_release.argtypes = [_P, _I64]
    L.pkv_bm_take_copies.restype = _I32
    L.pkv_bm_take_copies.argtypes = [_P, _P, _I32]
    L.pkv_bm_context_len.restype = _I32
    L.pkv_bm_context_len.argtypes = [_P, _I64]
    L.pkv_bm_table.restype = _I32
    L.pkv_bm_table.argtypes = [_P, _I64, _P, _I32]
    L.pkv_bm_export.restype = C.c_int
    L.pkv_bm_export.argtypes = [_P, _P, _I32, _P, _I32, _P]
    L.pkv_bm_stats.restype = C.c_int
    L.pkv_bm_stats.argtypes = [_P, _P, _I32]
    L.pkv_bm_ref.restype = _I32
    L.pkv_bm_ref.argtypes = [_P, _I32]
    L.pkv_bm_lru.restype = _I32
    L.pkv_bm_lru.argtypes = [_P, _P, _I32]


_setup(lib())

STATS = ("free", "evictable", "cached_keys", "sequences", "prompt_block_hits",
         "prompt_block_lookups", "evictions", "copies")


def _check(fn, st):
    if st == PKV_ENOSPACE:
        raise NoSpace(fn, st, lib().pkv_status_string(st).decode())
    if st < 0:
        raise PagedKVError(fn, st, lib().pkv_status_string(st).decode())
    return st


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, hash_namespace: int = 0):
        self._L = lib()
        self._h = self._L.pkv_bm_create(int(num_blocks), int(block_size), int(hash_namespace))
        if not self._h:
            raise ValueError("pkv_bm_create rejected the arguments")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            self._L.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add(self, seq: int, tokens) -> int:
        t = _i32(tokens)
        cached = C.c_int32(0)
        _check("pkv_bm_add", self._L.pkv_bm_add(self._h, int(seq), t.ctypes.data, t.size,
                                                C.byref(cached)))
        return cached.value

    def append(self, seq: int, tokens) -> None:
        t = _i32(tokens)
        _check("pkv_bm_append", self._L.pkv_bm_append(self._h, int(seq), t.ctypes.data if t.size
                                                      else None, t.size))

    def append_batch(self, seqs, token_start, tokens) -> int:
        """Appends tokens[token_start[i]:token_start[i+1]] to seqs[i] in order,
        stopping at the first failure; returns how many sequences were
        extended (raises if the first one fails)."""
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        ts, t = _i32(token_start), _i32(tokens)
        if ts.size != s.size + 1:
            raise ValueError("token_start must hold len(seqs) + 1 offsets")
        return _check("pkv_bm_append_batch",
                      self._L.pkv_bm_append_batch(self._h, s.ctypes.data, s.size, ts.ctypes.data,
                                                  t.ctypes.data if t.size else ts.ctypes.data))

    def fork(self, parent: int, child: int) -> None:
        _check("pkv_bm_fork", self._L.pkv_bm_fork(self._h, int(parent), int(child)))

    def release(self, seq: int) -> None:
        _check("pkv_bm_release", self._L.pkv_bm_release(self._h, int(seq)))

    def take_copies(self, max_copies: int = 1 << 16):
        out = np.empty(3 * max_copies, dtype=np.int32)
        n = _check("pkv_bm_take_copies",
                   self._L.pkv_bm_take_copies(self._h, out.ctypes.data, max_copies))
        return [tuple(int(x) for x in out[3 * i:3 * i + 3]) for i in range(n)]

    def context_len(self, seq: int) -> int:
        return _check("pkv_bm_context_len", self._L.pkv_bm_context_len(self._h, int(seq)))

    def table(self, seq: int, width: int = None):
        width = self.num_blocks if width is None else int(width)
        row = np.empty(width, dtype=np.int32)
        n = _check("pkv_bm_table", self._L.pkv_bm_table(self._h, int(seq), row.ctypes.data,
                                                        width))
        return [int(x) for x in row[:n]]

    def export(self, seqs, width: int):
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        tables = np.empty((s.size, width), dtype=np.int32)
        lens = np.empty(s.size, dtype=np.int32)
        _check("pkv_bm_export", self._L.pkv_bm_export(self._h, s.ctypes.data, s.size,
                                                      tables.ctypes.data, int(width),
                                                      lens.ctypes.data))
        return tables, lens

    def stats(self) -> dict:
        out = np.zeros(8, dtype=np.int64)
        _check("pkv_bm_stats", self._L.pkv_bm_stats(self._h, out.ctypes.data, 8))
        return dict(zip(STATS, (int(x) for x in out)))

    def ref(self, block: int) -> int:
        return _check("pkv_bm_ref", self._L.pkv_bm_ref(self._h, int(block)))

    def lru(self):
        n = _check("pkv_bm_lru", self._L.pkv_bm_lru(self._h, None, 0))
        out = np.empty(max(n, 1), dtype=np.int32)
        self._L.pkv_bm_lru(self._h, out.ctypes.data, n)
        return [int(x) for x in out[:n]]
