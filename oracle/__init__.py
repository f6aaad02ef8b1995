"""Python access to the CPU oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg
of bench.py may import this package.  The product path never does.

The oracle is plain C compiled by gcc into liboracle.so next to this file;
`build()` compiles it, `lib()` loads it (building it first if absent).
Array arguments are numpy arrays, passed by pointer.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = C.c_void_p
_I32 = C.c_int32
_I64 = C.c_int64
_F32 = C.c_float
_F64 = C.c_double


def build(extra_flags=()) -> str:
    """Compiles oracle.c with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", *extra_flags, "-o", _SO + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def lib():
    """Loads liboracle.so (building it if absent).  PKV_ORACLE_LIB names an
    alternative build of the same source, used by the planted-mistake test."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("PKV_ORACLE_LIB", _SO)
    if path == _SO and not os.path.exists(_SO):
        build()
    L = C.CDLL(path)
    sig = {
        "orc_kv_bytes_per_token": (_I64, [_I64, _I64, _I64, _I64]),
        "orc_kv_bytes_total": (_I64, [_I64, _I64, _I64, _I64, _I64, _I64]),
        "orc_bf16_value": (_F64, [C.c_uint16]),
        "orc_e4m3_value": (_F64, [C.c_uint8]),
        "orc_e4m3_encode": (C.c_uint8, [_F32]),
        "orc_e4m3_quantize": (C.c_uint8, [C.c_uint16, _F32]),
        "orc_check_tables": (_I32, [_P, _I32, _P, _I32, _I32, _I32]),
        "orc_append": (None, [_P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32,
                              _I32, _I32]),
        "orc_attend_range": (_F64, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                    _I32, _F64, _I32, _I32, _I32, _I32, _P]),
        "orc_lse_merge": (_F64, [_P, _P, _I32, _I32, _P]),
        "orc_paged_attention": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32,
                                       _I32, _I32, _I32, _F64, _I32, _I32, _P, _P, _P, _P]),
        "orc_split_reduce": (_I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P]),
        "orc_fp8_block_scales": (None, [_P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _P]),
        "orc_fp8_quantize_pool": (None, [_P, _P, _I32, _I32, _I32, _I32, _P]),
        "orc_int8_quantize": (C.c_uint8, [C.c_uint16, _F32, _F32]),
        "orc_fp8_wide_scales": (None, [_P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                       _P]),
        "orc_int8_block_params": (None, [_P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                         _P]),
        "orc_quantize_pool": (None, [_P, _P, _I32, _I32, _I32, _I32, _I32, _P]),
        "orc_gather_blocks": (None, [_P, _P, _I32, _I64, _P]),
        "orc_scatter_blocks": (None, [_P, _P, _I32, _I64, _P]),
        "orc_copy_blocks": (None, [_P, _P, _P, _I32, _I64]),
        "orc_write_tokens": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32,
                                    _I32, _I32, _I32]),
        "orc_multiquery_attention": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32,
                                            _I32, _I32, _I32, _I32, _F64, _P, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "need C-contiguous numpy"
    return a.ctypes.data


_DT = {"bf16": 0, "fp8": 1, "fp8_head": 2, "fp8_tensor": 3, "int8": 4,
       0: 0, 1: 1, 2: 2, 3: 3, 4: 4}


# ---------------------------------------------------------------- sizes
def kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes) -> int:
    return int(lib().orc_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def kv_bytes_total(layers, kv_heads, head_dim, seq_len, dtype_bytes, batch) -> int:
    return int(lib().orc_kv_bytes_total(layers, kv_heads, head_dim, seq_len, dtype_bytes,
                                        batch))


# ---------------------------------------------------------------- formats
def bf16_value(bits: int) -> float:
    return float(lib().orc_bf16_value(int(bits)))


def e4m3_value(code: int) -> float:
    return float(lib().orc_e4m3_value(int(code)))


def e4m3_encode(y: float) -> int:
    return int(lib().orc_e4m3_encode(float(np.float32(y))))


def e4m3_quantize(bits: int, scale) -> int:
    return int(lib().orc_e4m3_quantize(int(bits), float(np.float32(scale))))


def e4m3_quantize_array(bits: np.ndarray, scale) -> np.ndarray:
    """Elementwise quantise of bf16 bits with one scale (a 1-block pool)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    flat = bits.reshape(1, 1, 1, -1)
    sc = np.asarray([scale], dtype=np.float32)
    out = np.empty(flat.shape, dtype=np.uint8)
    lib().orc_fp8_quantize_pool(_ptr(flat), _ptr(sc), 1, 1, 1, flat.shape[-1], _ptr(out))
    return out.reshape(bits.shape)


# ---------------------------------------------------------------- tables
def check_tables(block_tables, context_lens, block_size, num_blocks) -> int:
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    return int(lib().orc_check_tables(_ptr(bt), bt.shape[1], _ptr(cl), cl.shape[0],
                                      block_size, num_blocks))


# ---------------------------------------------------------------- append
def append(k_new, v_new, k_cache, v_cache, block_tables, context_lens, block_size,
           kv_dtype="bf16", k_scale=None, v_scale=None) -> None:
    """In-place scatter of the new token into host copies of the pools."""
    B, Hkv, D = k_new.shape
    lib().orc_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                     _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), block_tables.shape[1],
                     _ptr(context_lens), B, Hkv, D, block_size, _DT[kv_dtype])


# ---------------------------------------------------------------- attention
def attend_range(query, k_cache, v_cache, block_tables, b, hq, t0, t1, scale, *,
                 block_size, Hkv, kv_dtype="bf16", k_scale=None, v_scale=None):
    """(out[D] float64, lse) of query head hq of sequence b over [t0, t1)."""
    B, Hq, D = query.shape
    out = np.empty(D, dtype=np.float64)
    lse = lib().orc_attend_range(_ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                 _ptr(v_scale), _ptr(block_tables), block_tables.shape[1],
                                 Hq, Hkv, D, block_size, _DT[kv_dtype], float(scale),
                                 int(b), int(hq), int(t0), int(t1), _ptr(out))
    return out, float(lse)


def paged_attention(query, k_cache, v_cache, block_tables, context_lens, scale, *,
                    block_size, Hkv, kv_dtype="bf16", k_scale=None, v_scale=None,
                    split_tokens=0, max_splits=0, want_partials=False):
    """Whole-batch oracle.  Returns (out [B,Hq,D], lse [B,Hq]) in float64,
    plus (partial_out [B,Hq,max_splits,D], partial_lse [B,Hq,max_splits])
    when want_partials (entries past a sequence's last split are NaN)."""
    B, Hq, D = query.shape
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    po = pl = None
    if want_partials:
        assert split_tokens > 0
        po = np.full((B, Hq, max_splits, D), np.nan)
        pl = np.full((B, Hq, max_splits), np.nan)
    rc = lib().orc_paged_attention(_ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                   _ptr(v_scale), _ptr(block_tables), block_tables.shape[1],
                                   _ptr(context_lens), B, Hq, Hkv, D, block_size,
                                   _DT[kv_dtype], float(scale), int(split_tokens),
                                   int(max_splits), _ptr(out), _ptr(lse), _ptr(po), _ptr(pl))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    if want_partials:
        return out, lse, po, pl
    return out, lse


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, D = o_parts.shape
    out = np.empty(D, dtype=np.float64)
    lse = lib().orc_lse_merge(_ptr(o_parts), _ptr(lse_parts), n, D, _ptr(out))
    return out, float(lse)


def split_reduce(partial_out, partial_lse, context_lens, split_tokens):
    B, Hq, max_splits, D = partial_out.shape
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = lib().orc_split_reduce(_ptr(partial_out), _ptr(partial_lse), _ptr(context_lens),
                                B, Hq, D, split_tokens, max_splits, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, lse


# ---------------------------------------------------------------- fp8 pools
def fp8_block_scales(src_pool, block_tables, context_lens, block_size):
    nb, bs, Hkv, D = src_pool.shape
    sc = np.empty((nb, Hkv), dtype=np.float32)
    lib().orc_fp8_block_scales(_ptr(src_pool), _ptr(block_tables), block_tables.shape[1],
                               _ptr(context_lens), context_lens.shape[0], Hkv, D, block_size,
                               nb, _ptr(sc))
    return sc


def fp8_quantize_pool(src_pool, scales):
    nb, bs, Hkv, D = src_pool.shape
    codes = np.empty(src_pool.shape, dtype=np.uint8)
    lib().orc_fp8_quantize_pool(_ptr(src_pool), _ptr(scales), nb, bs, Hkv, D, _ptr(codes))
    return codes


# ---------------------------------------------------------------- several new tokens
def write_tokens(k_rows, v_rows, query_start, k_cache, v_cache, block_tables, context_lens,
                 block_size, kv_dtype="bf16", k_scale=None, v_scale=None) -> None:
    """In-place write of each sequence's q_b new K/V rows ([total_rows, Hkv, D])
    into the positions T_b - q_b .. T_b - 1 of host copies of the pools."""
    total, Hkv, D = k_rows.shape
    B = context_lens.shape[0]
    rc = lib().orc_write_tokens(_ptr(k_rows), _ptr(v_rows), _ptr(query_start), _ptr(k_cache),
                                _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                B, Hkv, D, block_size, _DT[kv_dtype])
    if rc != 0:
        raise ValueError("oracle rejected the arguments")


def multiquery_attention(query, query_start, k_cache, v_cache, block_tables, context_lens,
                         scale, *, block_size, Hkv, kv_dtype="bf16", k_scale=None,
                         v_scale=None):
    """Causal multi-query oracle: (out [total_rows, Hq, D], lse [total_rows, Hq])."""
    total, Hq, D = query.shape
    B = context_lens.shape[0]
    out = np.empty((total, Hq, D), dtype=np.float64)
    lse = np.empty((total, Hq), dtype=np.float64)
    rc = lib().orc_multiquery_attention(_ptr(query), _ptr(query_start), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                        _ptr(block_tables), block_tables.shape[1],
                                        _ptr(context_lens), B, Hq, Hkv, D, block_size,
                                        _DT[kv_dtype], float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, lse


# ---------------------------------------------------------------- whole blocks
def _block_bytes(pool):
    return int(pool[0].nbytes) if pool.shape[0] else 0


def gather_blocks(pool, ids):
    """pool [num_blocks, ...] -> [n, ...] with out[i] = pool[ids[i]]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    out = np.empty((ids.size,) + pool.shape[1:], dtype=pool.dtype)
    lib().orc_gather_blocks(_ptr(pool), _ptr(ids), ids.size, _block_bytes(pool), _ptr(out))
    return out


def scatter_blocks(blocks, ids, pool):
    """In place: pool[ids[i]] = blocks[i]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    lib().orc_scatter_blocks(_ptr(blocks), _ptr(ids), ids.size, _block_bytes(pool), _ptr(pool))


def copy_blocks(pool, src, dst):
    """In place: pool[dst[i]] = pool[src[i]]."""
    src = np.ascontiguousarray(src, dtype=np.int32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    lib().orc_copy_blocks(_ptr(pool), _ptr(src), _ptr(dst), src.size, _block_bytes(pool))


# ---------------------------------------------------------------- other 1-byte formats
def int8_quantize(x_bf16: int, scale: float, zero_point: float) -> int:
    return int(lib().orc_int8_quantize(int(x_bf16), float(scale), float(zero_point)))


def fp8_wide_scales(src_bf16, block_tables, context_lens, block_size, per_tensor=False):
    """E4M3 scales per kv head ([Hkv]) or per tensor ([1])."""
    nb, _, Hkv, D = src_bf16.shape
    out = np.empty(1 if per_tensor else Hkv, dtype=np.float32)
    lib().orc_fp8_wide_scales(_ptr(src_bf16), _ptr(block_tables), block_tables.shape[1],
                              _ptr(context_lens), context_lens.shape[0], Hkv, D, block_size,
                              nb, int(bool(per_tensor)), _ptr(out))
    return out


def int8_block_params(src_bf16, block_tables, context_lens, block_size, symmetric=False):
    """[num_blocks, Hkv, 2] (scale, zero point) pairs."""
    nb, _, Hkv, D = src_bf16.shape
    out = np.empty((nb, Hkv, 2), dtype=np.float32)
    lib().orc_int8_block_params(_ptr(src_bf16), _ptr(block_tables), block_tables.shape[1],
                                _ptr(context_lens), context_lens.shape[0], Hkv, D, block_size,
                                nb, int(bool(symmetric)), _ptr(out))
    return out


def quantize_pool(src_bf16, scales, kv_dtype):
    """A bf16 pool quantised to 1-byte codes of kv_dtype ("fp8", "fp8_head",
    "fp8_tensor", "int8")."""
    nb, bs, Hkv, D = src_bf16.shape
    out = np.empty(src_bf16.shape, dtype=np.uint8)
    lib().orc_quantize_pool(_ptr(src_bf16), _ptr(np.ascontiguousarray(scales, np.float32)),
                            _DT[kv_dtype], nb, bs, Hkv, D, _ptr(out))
    return out
