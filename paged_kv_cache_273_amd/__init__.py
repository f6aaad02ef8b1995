"""Paged decode attention for AMD Instinct MI355X (gfx950).

Thin Python binding of libpagedkv.so (C ABI in include/pagedkv.h).  Every
step of the computation runs in the HIP kernels of that library; this
module only turns torch tensors into pointers and sizes.  PyTorch provides
device memory and streams, nothing else.  If the library is missing the
import fails: there is no fallback.

Entry points (same names as the C ABI):
    paged_kv_append(...)          write the step's new K/V rows into the cache
    paged_decode_attention(...)   attention of one query per sequence over
                                  its block-table-gathered cache
    split_context_reduce(...)     log-sum-exp merge of split-context partials
    paged_decode_attention_balanced(...)  the decode attention, work-balanced
    paged_append_decode_attention(...), paged_append_decode_attention_balanced(...)
                                  append and decode attention in one launch
    paged_kv_write(...)           several new K/V rows per sequence
    paged_multiquery_attention(...)  causal attention of several new tokens
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ELAUNCH, PKV_ENOSPACE, PKV_ENOMEM = 0, -1, -2, -3, -4, -5
PKV_BF16, PKV_FP8_E4M3, PKV_FP8_E4M3_PER_HEAD, PKV_FP8_E4M3_PER_TENSOR, PKV_INT8 = 0, 1, 2, 3, 4
KV_DTYPES = {"bf16": PKV_BF16, "fp8": PKV_FP8_E4M3, "fp8_head": PKV_FP8_E4M3_PER_HEAD,
             "fp8_tensor": PKV_FP8_E4M3_PER_TENSOR, "int8": PKV_INT8}

EXPORTS = ("paged_kv_append", "paged_decode_attention", "split_context_reduce",
           "paged_decode_attention_balanced", "paged_decode_workspace_size",
           "paged_append_decode_attention", "paged_append_decode_attention_balanced",
           "paged_kv_write", "paged_multiquery_attention", "paged_multiquery_workspace_size",
           "pkv_status_string", "paged_kv_gather_blocks", "paged_kv_scatter_blocks",
           "paged_kv_copy_blocks", "paged_decode_attention_balanced_noalloc",
           # host block manager (include/pkv_block_manager.h; binding in block_manager.py)
           "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_add", "pkv_bm_append",
           "pkv_bm_append_batch", "pkv_bm_fork",
           "pkv_bm_release", "pkv_bm_take_copies", "pkv_bm_context_len", "pkv_bm_table",
           "pkv_bm_export", "pkv_bm_stats", "pkv_bm_ref", "pkv_bm_lru",
           # measurement probe (include/pkv_probe.h)
           "pkv_stream_read")


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{LIB_PATH} is not built: run __graft_entry__.build() "
            "(or python paged_kv_cache_273_amd/_build.py) first")
    L = C.CDLL(path)
    P, I = C.c_void_p, C.c_int32
    L.paged_kv_append.restype = C.c_int
    L.paged_kv_append.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, P]
    L.paged_decode_attention.restype = C.c_int
    L.paged_decode_attention.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, C.c_float,
                                         I, P, P, P, I, P, P]
    L.paged_append_decode_attention.restype = C.c_int
    L.paged_append_decode_attention.argtypes = [P, P, P] + L.paged_decode_attention.argtypes[1:]
    L.split_context_reduce.restype = C.c_int
    L.split_context_reduce.argtypes = [P, P, P, I, I, I, I, I, P, P, P]
    L.paged_decode_attention_balanced.restype = C.c_int
    L.paged_decode_attention_balanced.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, I, I,
                                                  C.c_float, P, C.c_int64, P, P, P]
    L.paged_decode_attention_balanced_noalloc.restype = C.c_int
    L.paged_decode_attention_balanced_noalloc.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I,
                                                          I, I, I, C.c_float, P, P, P]
    L.paged_append_decode_attention_balanced.restype = C.c_int
    L.paged_append_decode_attention_balanced.argtypes = (
        [P, P, P] + L.paged_decode_attention_balanced.argtypes[1:])
    L.paged_decode_workspace_size.restype = C.c_int64
    L.paged_decode_workspace_size.argtypes = [I, I, I, I, I]
    L.paged_kv_write.restype = C.c_int
    L.paged_kv_write.argtypes = [P, P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, P]
    L.paged_multiquery_attention.restype = C.c_int
    L.paged_multiquery_attention.argtypes = [P, P, I, I, P, P, P, P, P, I, P, I, I, I, I, I, I,
                                             I, C.c_float, P, C.c_int64, P, P, P]
    L.paged_multiquery_workspace_size.restype = C.c_int64
    L.paged_multiquery_workspace_size.argtypes = [I, I, I, I, I, I]
    for name in ("paged_kv_gather_blocks", "paged_kv_scatter_blocks"):
        getattr(L, name).restype = C.c_int
        getattr(L, name).argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P]
    L.paged_kv_copy_blocks.restype = C.c_int
    L.paged_kv_copy_blocks.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P]
    L.pkv_stream_read.restype = C.c_int
    L.pkv_stream_read.argtypes = [P, C.c_int64, I, P, P]
    L.pkv_status_string.restype = C.c_char_p
    L.pkv_status_string.argtypes = [C.c_int]
    return L


_lib = _load()


def lib():
    return _lib


def _check(fn: str, status: int) -> None:
    if status != PKV_OK:
        raise PagedKVError(fn, status, _lib.pkv_status_string(status).decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


_BF16_BITS = (torch.bfloat16, torch.int16, torch.uint16)
_FP8_CODES = (torch.uint8, torch.float8_e4m3fn)


def _kv_dtype(cache: torch.Tensor, kv_dtype=None) -> int:
    """The cache format: given (a pkv_dtype code or a name of KV_DTYPES), or
    inferred from the tensor (bf16 bits, or E4M3FN codes with per-(block,
    kv head) scales)."""
    if kv_dtype is not None:
        code = KV_DTYPES.get(kv_dtype, kv_dtype)
        one_byte = cache.dtype in _FP8_CODES or cache.dtype == torch.int8
        if (code == PKV_BF16) == one_byte or code not in KV_DTYPES.values():
            raise TypeError(f"cache dtype {cache.dtype} does not hold kv_dtype {kv_dtype!r}")
        return code
    if cache.dtype in _BF16_BITS:
        return PKV_BF16
    if cache.dtype in _FP8_CODES:
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported cache dtype {cache.dtype}")


def _need(t: torch.Tensor, dtypes, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")


# Shape checks.  The C ABI receives one B, Hq, Hkv, D, block size and split
# count per call and cannot see the tensors, so a tensor whose shape
# disagrees with them would be read or written out of bounds on the device.
# Every tensor is checked here, before any pointer is taken.
def _shape(t, shape, name, dtypes=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if dtypes is not None:
        _need(t, dtypes, name)
    elif not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dim() != len(shape) or any(w is not None and int(n) != w
                                    for n, w in zip(t.shape, shape)):
        want = tuple("*" if w is None else w for w in shape)
        raise ValueError(f"{name}: shape {tuple(t.shape)} does not match {want}")


def _same_device(ref, **ts):
    for name, t in ts.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the call's tensors on {ref.device}")


def _scale_shape(code, nb, Hkv):
    return {PKV_FP8_E4M3: (nb, Hkv), PKV_FP8_E4M3_PER_HEAD: (Hkv,),
            PKV_FP8_E4M3_PER_TENSOR: (1,), PKV_INT8: (nb, Hkv, 2)}.get(code)


def _cache_args(k_cache, v_cache, k_scale, v_scale, kv_dtype):
    """Checks a K/V cache pair and its scales; returns (num_blocks,
    block_size, Hkv, D, pkv_dtype code)."""
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4:
        raise ValueError("k_cache must be a [num_blocks, block_size, Hkv, D] tensor")
    nb, bs, Hkv, D = (int(n) for n in k_cache.shape)
    code = _kv_dtype(k_cache, kv_dtype)
    _shape(v_cache, (nb, bs, Hkv, D), "v_cache")
    if v_cache.element_size() != k_cache.element_size():
        raise TypeError(f"v_cache dtype {v_cache.dtype} differs from k_cache {k_cache.dtype}")
    sc = _scale_shape(code, nb, Hkv)
    if sc is not None:
        _shape(k_scale, sc, "k_scale", (torch.float32,))
        _shape(v_scale, sc, "v_scale", (torch.float32,))
    _same_device(k_cache, v_cache=v_cache, k_scale=k_scale if sc else None,
                 v_scale=v_scale if sc else None)
    return nb, bs, Hkv, D, code


def _table_args(block_tables, context_lens, B):
    """Checks block_tables [B, max_blocks] and context_lens [B] (int32);
    returns max_blocks."""
    _shape(block_tables, (B, None), "block_tables", (torch.int32,))
    _shape(context_lens, (B,), "context_lens", (torch.int32,))
    return int(block_tables.shape[1])


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def paged_kv_append(k_new, v_new, k_cache, v_cache, block_tables, context_lens, *,
                    k_scale=None, v_scale=None, kv_dtype=None, stream=None) -> None:
    """k_new/v_new [B, Hkv, D] bf16; caches [num_blocks, block_size, Hkv, D]
    (bf16 bits or E4M3FN codes); block_tables [B, max_blocks] int32;
    context_lens [B] int32 (including the new token)."""
    nb, bs, Hkv, D, code = _cache_args(k_cache, v_cache, k_scale, v_scale, kv_dtype)
    _shape(k_new, (None, Hkv, D), "k_new", _BF16_BITS)
    B = int(k_new.shape[0])
    _shape(v_new, (B, Hkv, D), "v_new", _BF16_BITS)
    max_blocks = _table_args(block_tables, context_lens, B)
    _same_device(k_cache, k_new=k_new, v_new=v_new, block_tables=block_tables,
                 context_lens=context_lens)
    st = _lib.paged_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                              _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                              max_blocks, _ptr(context_lens), B, Hkv, D, bs, nb,
                              code, _stream(stream))
    _check("paged_kv_append", st)


def _decode(name, query, new, k_cache, v_cache, block_tables, context_lens, scale, out,
            lse_out, split_tokens, partial_out, partial_lse, k_scale, v_scale, kv_dtype, stream):
    nb, bs, Hkv, D, code = _cache_args(k_cache, v_cache, k_scale, v_scale, kv_dtype)
    _shape(query, (None, None, D), "query", _BF16_BITS)
    B, Hq = int(query.shape[0]), int(query.shape[1])
    max_blocks = _table_args(block_tables, context_lens, B)
    _new_row_args(new, B, Hkv, D)
    max_splits = 0
    if split_tokens == 0:
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
        _shape(out, (B, Hq, D), "out", (torch.float32,))
    else:
        if partial_out is None or partial_lse is None:
            raise ValueError("split mode needs partial_out and partial_lse")
        _shape(partial_out, (B, Hq, None, D), "partial_out", (torch.float32,))
        max_splits = int(partial_out.shape[2])
        _shape(partial_lse, (B, Hq, max_splits), "partial_lse", (torch.float32,))
    if lse_out is not None:
        _shape(lse_out, (B, Hq), "lse_out", (torch.float32,))
    _same_device(k_cache, query=query, block_tables=block_tables, context_lens=context_lens,
                 out=out, lse_out=lse_out, partial_out=partial_out, partial_lse=partial_lse)
    st = getattr(_lib, name)(
        _ptr(query), *_new_rows(new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(block_tables), max_blocks, _ptr(context_lens), B, Hq,
        Hkv, D, bs, nb, code, float(scale), int(split_tokens),
        _ptr(out), _ptr(partial_out), _ptr(partial_lse), max_splits, _ptr(lse_out),
        _stream(stream))
    _check(name, st)
    return out if split_tokens == 0 else (partial_out, partial_lse)


def _new_row_args(new, B, Hkv, D):
    if new is not None:
        _shape(new[0], (B, Hkv, D), "k_new", _BF16_BITS)
        _shape(new[1], (B, Hkv, D), "v_new", _BF16_BITS)


def _new_rows(new):
    if new is None:
        return ()
    k_new, v_new = new
    return (_ptr(k_new), _ptr(v_new))


def paged_decode_attention(query, k_cache, v_cache, block_tables, context_lens, scale, *,
                           out=None, lse_out=None, split_tokens=0, partial_out=None,
                           partial_lse=None, k_scale=None, v_scale=None, kv_dtype=None,
                           stream=None):
    """query [B, Hq, D] bf16.  split_tokens == 0: writes out [B, Hq, D] float32
    (and lse_out [B, Hq]) and returns out.  split_tokens > 0: writes
    partial_out [B, Hq, max_splits, D] / partial_lse [B, Hq, max_splits] and
    returns them (combine with split_context_reduce)."""
    return _decode("paged_decode_attention", query, None, k_cache, v_cache, block_tables,
                   context_lens, scale, out, lse_out, split_tokens, partial_out, partial_lse,
                   k_scale, v_scale, kv_dtype, stream)


def paged_append_decode_attention(query, k_new, v_new, k_cache, v_cache, block_tables,
                                  context_lens, scale, *, out=None, lse_out=None,
                                  split_tokens=0, partial_out=None, partial_lse=None,
                                  k_scale=None, v_scale=None, kv_dtype=None, stream=None):
    """paged_kv_append(k_new, v_new, ...) then paged_decode_attention(...),
    in one launch; k_new / v_new [B, Hkv, D] bf16."""
    return _decode("paged_append_decode_attention", query, (k_new, v_new), k_cache, v_cache,
                   block_tables, context_lens, scale, out, lse_out, split_tokens, partial_out,
                   partial_lse, k_scale, v_scale, kv_dtype, stream)


def paged_decode_workspace_size(Hq, Hkv, D, block_size, kv_dtype=PKV_BF16) -> int:
    """Bytes of workspace paged_decode_attention_balanced needs on the
    current device."""
    n = int(_lib.paged_decode_workspace_size(Hq, Hkv, D, block_size, kv_dtype))
    if n < 0:
        _check("paged_decode_workspace_size", n)
    return n


def make_workspace(query, k_cache, kv_dtype=None) -> torch.Tensor:
    """A device buffer large enough for paged_decode_attention_balanced."""
    B, Hq, D = query.shape
    n = paged_decode_workspace_size(Hq, k_cache.shape[2], D, k_cache.shape[1],
                                    _kv_dtype(k_cache, kv_dtype))
    return torch.empty(n, dtype=torch.uint8, device=query.device)


def _balanced(name, query, new, k_cache, v_cache, block_tables, context_lens, scale, workspace,
              out, lse_out, k_scale, v_scale, kv_dtype, stream):
    nb, bs, Hkv, D, code = _cache_args(k_cache, v_cache, k_scale, v_scale, kv_dtype)
    _shape(query, (None, None, D), "query", _BF16_BITS)
    B, Hq = int(query.shape[0]), int(query.shape[1])
    max_blocks = _table_args(block_tables, context_lens, B)
    _new_row_args(new, B, Hkv, D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=query.device)
    _shape(out, (B, Hq, D), "out", (torch.float32,))
    if lse_out is not None:
        _shape(lse_out, (B, Hq), "lse_out", (torch.float32,))
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace: expected a torch.Tensor")
    _same_device(k_cache, query=query, block_tables=block_tables, context_lens=context_lens,
                 out=out, lse_out=lse_out, workspace=workspace)
    nbytes = workspace.numel() * workspace.element_size()
    st = getattr(_lib, name)(
        _ptr(query), *_new_rows(new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(block_tables), max_blocks, _ptr(context_lens), B, Hq,
        Hkv, D, bs, nb, code, float(scale), _ptr(workspace), nbytes,
        _ptr(out), _ptr(lse_out), _stream(stream))
    _check(name, st)
    return out


def paged_decode_attention_balanced(query, k_cache, v_cache, block_tables, context_lens, scale,
                                    *, workspace, out=None, lse_out=None, k_scale=None,
                                    v_scale=None, kv_dtype=None, stream=None):
    """Single-pass paged decode attention with the work of all (sequence,
    kv head) pairs cut into equal ranges (for ragged batches).  workspace:
    a device buffer of paged_decode_workspace_size(...) bytes."""
    return _balanced("paged_decode_attention_balanced", query, None, k_cache, v_cache,
                     block_tables, context_lens, scale, workspace, out, lse_out, k_scale,
                     v_scale, kv_dtype, stream)


def paged_append_decode_attention_balanced(query, k_new, v_new, k_cache, v_cache,
                                           block_tables, context_lens, scale, *, workspace,
                                           out=None, lse_out=None, k_scale=None,
                                           v_scale=None, kv_dtype=None, stream=None):
    """paged_kv_append(k_new, v_new, ...) then
    paged_decode_attention_balanced(...), in one launch."""
    return _balanced("paged_append_decode_attention_balanced", query, (k_new, v_new), k_cache,
                     v_cache, block_tables, context_lens, scale, workspace, out, lse_out,
                     k_scale, v_scale, kv_dtype, stream)


def paged_decode_attention_balanced_noalloc(query, k_cache, v_cache, block_tables,
                                            context_lens, scale, *, out, lse_out=None,
                                            k_scale=None, v_scale=None, kv_dtype=None,
                                            stream=None):
    """paged_decode_attention_balanced without a workspace argument: the
    library's static per-GPU scratch array serves as the workspace, so the
    call allocates nothing (for callers that cannot allocate).  `out` must
    be given.  Calls that may overlap on one GPU race."""
    nb, bs, Hkv, D, code = _cache_args(k_cache, v_cache, k_scale, v_scale, kv_dtype)
    _shape(query, (None, None, D), "query", _BF16_BITS)
    B, Hq = int(query.shape[0]), int(query.shape[1])
    max_blocks = _table_args(block_tables, context_lens, B)
    _shape(out, (B, Hq, D), "out", (torch.float32,))
    if lse_out is not None:
        _shape(lse_out, (B, Hq), "lse_out", (torch.float32,))
    _same_device(k_cache, query=query, block_tables=block_tables, context_lens=context_lens,
                 out=out, lse_out=lse_out)
    st = _lib.paged_decode_attention_balanced_noalloc(
        _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), max_blocks, _ptr(context_lens), B, Hq, Hkv, D, bs, nb, code,
        float(scale), _ptr(out), _ptr(lse_out), _stream(stream))
    _check("paged_decode_attention_balanced_noalloc", st)
    return out


def split_context_reduce(partial_out, partial_lse, context_lens, split_tokens, *, out=None,
                         lse_out=None, stream=None):
    """Merges partials [B, Hq, max_splits, D] into out [B, Hq, D] float32."""
    _shape(partial_out, (None, None, None, None), "partial_out", (torch.float32,))
    B, Hq, ms, D = (int(n) for n in partial_out.shape)
    _shape(partial_lse, (B, Hq, ms), "partial_lse", (torch.float32,))
    _shape(context_lens, (B,), "context_lens", (torch.int32,))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=partial_out.device)
    _shape(out, (B, Hq, D), "out", (torch.float32,))
    if lse_out is not None:
        _shape(lse_out, (B, Hq), "lse_out", (torch.float32,))
    _same_device(partial_out, partial_lse=partial_lse, context_lens=context_lens, out=out,
                 lse_out=lse_out)
    st = _lib.split_context_reduce(_ptr(partial_out), _ptr(partial_lse), _ptr(context_lens), B,
                                   Hq, D, int(split_tokens), ms, _ptr(out), _ptr(lse_out),
                                   _stream(stream))
    _check("split_context_reduce", st)
    return out


def paged_kv_write(k_rows, v_rows, query_start, k_cache, v_cache, block_tables, context_lens,
                   max_query_len, *, k_scale=None, v_scale=None, kv_dtype=None,
                   stream=None) -> None:
    """k_rows/v_rows [rows, Hkv, D] bf16: rows query_start[b] + i go to
    positions context_lens[b] - q_b + i (q_b = query_start[b+1] -
    query_start[b] <= max_query_len)."""
    nb, bs, Hkv, D, code = _cache_args(k_cache, v_cache, k_scale, v_scale, kv_dtype)
    _shape(k_rows, (None, Hkv, D), "k_rows", _BF16_BITS)
    _shape(v_rows, tuple(k_rows.shape), "v_rows", _BF16_BITS)
    _shape(context_lens, (None,), "context_lens", (torch.int32,))
    B = int(context_lens.shape[0])
    _shape(query_start, (B + 1,), "query_start (B + 1 offsets)", (torch.int32,))
    max_blocks = _table_args(block_tables, context_lens, B)
    _same_device(k_cache, k_rows=k_rows, v_rows=v_rows, query_start=query_start,
                 block_tables=block_tables, context_lens=context_lens)
    st = _lib.paged_kv_write(_ptr(k_rows), _ptr(v_rows), _ptr(query_start), _ptr(k_cache),
                             _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                             max_blocks, _ptr(context_lens), B, int(max_query_len),
                             Hkv, D, bs, nb, code, _stream(stream))
    _check("paged_kv_write", st)


def paged_multiquery_workspace_size(Hq, Hkv, D, block_size, max_query_len,
                                    kv_dtype=PKV_BF16) -> int:
    """Bytes of workspace paged_multiquery_attention needs on the current
    device."""
    n = int(_lib.paged_multiquery_workspace_size(Hq, Hkv, D, block_size, kv_dtype,
                                                 int(max_query_len)))
    if n < 0:
        _check("paged_multiquery_workspace_size", n)
    return n


def make_multiquery_workspace(query, k_cache, max_query_len, kv_dtype=None) -> torch.Tensor:
    """A device buffer large enough for paged_multiquery_attention."""
    _, Hq, D = query.shape
    n = paged_multiquery_workspace_size(Hq, k_cache.shape[2], D, k_cache.shape[1],
                                        max_query_len, _kv_dtype(k_cache, kv_dtype))
    return torch.empty(n, dtype=torch.uint8, device=query.device)


def paged_multiquery_attention(query, query_start, k_cache, v_cache, block_tables, context_lens,
                               scale, max_query_len, *, workspace, out=None, lse_out=None,
                               k_scale=None, v_scale=None, kv_dtype=None, stream=None):
    """query [rows, Hq, D] bf16: row query_start[b] + i (position
    context_lens[b] - q_b + i) attends causally over its sequence's tokens
    up to its own position.  Writes out [rows, Hq, D] float32 (and lse_out
    [rows, Hq]) and returns out."""
    nb, bs, Hkv, D, code = _cache_args(k_cache, v_cache, k_scale, v_scale, kv_dtype)
    _shape(query, (None, None, D), "query", _BF16_BITS)
    rows, Hq = int(query.shape[0]), int(query.shape[1])
    _shape(context_lens, (None,), "context_lens", (torch.int32,))
    B = int(context_lens.shape[0])
    _shape(query_start, (B + 1,), "query_start (B + 1 offsets)", (torch.int32,))
    max_blocks = _table_args(block_tables, context_lens, B)
    if out is None:
        out = torch.empty((rows, Hq, D), dtype=torch.float32, device=query.device)
    _shape(out, (rows, Hq, D), "out", (torch.float32,))
    if lse_out is not None:
        _shape(lse_out, (rows, Hq), "lse_out", (torch.float32,))
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace: expected a torch.Tensor")
    _same_device(k_cache, query=query, query_start=query_start, block_tables=block_tables,
                 context_lens=context_lens, out=out, lse_out=lse_out, workspace=workspace)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.paged_multiquery_attention(
        _ptr(query), _ptr(query_start), rows, int(max_query_len), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), max_blocks,
        _ptr(context_lens), B, Hq, Hkv, D, bs, nb, code, float(scale),
        _ptr(workspace), nbytes, _ptr(out), _ptr(lse_out), _stream(stream))
    _check("paged_multiquery_attention", st)
    return out


def _any_ptr(t):
    """Pointer of a device tensor or of a pinned host tensor (both are
    addressable by the kernels)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError("host buffers must be pinned (pin_memory=True)")
    return t.data_ptr()


def _move_shape(k_cache, kv_dtype=None):
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4:
        raise ValueError("k_cache must be a [num_blocks, block_size, Hkv, D] tensor")
    nb, bs, Hkv, D = (int(n) for n in k_cache.shape)
    return nb, bs, Hkv, D, _kv_dtype(k_cache, kv_dtype)


def _block_buffers(k_cache, v_cache, n, bufs, scales, code):
    """Checks the pool pair and the [n, block_size, Hkv, D] block buffers
    (and, for formats with per-block scales, [n, Hkv] / [n, Hkv, 2] scale
    buffers) of a block move."""
    nb, bs, Hkv, D = (int(x) for x in k_cache.shape)
    _shape(v_cache, (nb, bs, Hkv, D), "v_cache")
    for name, t in bufs.items():
        _shape(t, (n, bs, Hkv, D), name)
        if t.element_size() != k_cache.element_size():
            raise TypeError(f"{name}: dtype {t.dtype} differs from the cache's {k_cache.dtype}")
    per_block = {PKV_FP8_E4M3: (Hkv,), PKV_INT8: (Hkv, 2)}.get(code)
    for name, (t, rows) in scales.items():
        if per_block is not None:
            _shape(t, (rows,) + per_block, name, (torch.float32,))


def paged_kv_gather_blocks(k_cache, v_cache, block_ids, k_out, v_out, *, k_scale=None,
                           v_scale=None, k_scale_out=None, v_scale_out=None, kv_dtype=None,
                           stream=None):
    """k_out[i] = k_cache[block_ids[i]] (and V, and fp8 scales).  Outputs may
    be pinned host tensors (swap out / offload)."""
    _shape(block_ids, (None,), "block_ids", (torch.int32,))
    nb, bs, Hkv, D, dt = _move_shape(k_cache, kv_dtype)
    n = int(block_ids.shape[0])
    _block_buffers(k_cache, v_cache, n, {"k_out": k_out, "v_out": v_out},
                   {"k_scale": (k_scale, nb), "v_scale": (v_scale, nb),
                    "k_scale_out": (k_scale_out, n), "v_scale_out": (v_scale_out, n)}, dt)
    st = _lib.paged_kv_gather_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _any_ptr(block_ids),
        block_ids.numel(), bs, Hkv, D, nb, dt, _any_ptr(k_out), _any_ptr(v_out),
        _any_ptr(k_scale_out), _any_ptr(v_scale_out), _stream(stream))
    _check("paged_kv_gather_blocks", st)


def paged_kv_scatter_blocks(k_in, v_in, block_ids, k_cache, v_cache, *, k_scale_in=None,
                            v_scale_in=None, k_scale=None, v_scale=None, kv_dtype=None,
                            stream=None):
    """k_cache[block_ids[i]] = k_in[i] (and V, and fp8 scales).  Inputs may be
    pinned host tensors (swap in)."""
    _shape(block_ids, (None,), "block_ids", (torch.int32,))
    nb, bs, Hkv, D, dt = _move_shape(k_cache, kv_dtype)
    n = int(block_ids.shape[0])
    _block_buffers(k_cache, v_cache, n, {"k_in": k_in, "v_in": v_in},
                   {"k_scale": (k_scale, nb), "v_scale": (v_scale, nb),
                    "k_scale_in": (k_scale_in, n), "v_scale_in": (v_scale_in, n)}, dt)
    st = _lib.paged_kv_scatter_blocks(
        _any_ptr(k_in), _any_ptr(v_in), _any_ptr(k_scale_in), _any_ptr(v_scale_in),
        _any_ptr(block_ids), block_ids.numel(), bs, Hkv, D, nb, dt, _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _stream(stream))
    _check("paged_kv_scatter_blocks", st)


def paged_kv_copy_blocks(k_cache, v_cache, src_ids, dst_ids, *, k_scale=None, v_scale=None,
                         kv_dtype=None, stream=None):
    """k_cache[dst_ids[i]] = k_cache[src_ids[i]] (copy-on-write copies)."""
    _shape(src_ids, (None,), "src_ids", (torch.int32,))
    _shape(dst_ids, (int(src_ids.shape[0]),), "dst_ids", (torch.int32,))
    nb, bs, Hkv, D, dt = _move_shape(k_cache, kv_dtype)
    _block_buffers(k_cache, v_cache, 0, {}, {"k_scale": (k_scale, nb), "v_scale": (v_scale, nb)},
                   dt)
    st = _lib.paged_kv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                   _any_ptr(src_ids), _any_ptr(dst_ids), src_ids.numel(), bs, Hkv,
                                   D, nb, dt, _stream(stream))
    _check("paged_kv_copy_blocks", st)


def max_splits_for(max_context: int, split_tokens: int) -> int:
    """Number of partial slots a sequence of max_context tokens needs."""
    return max(1, (int(max_context) + split_tokens - 1) // split_tokens)


def pkv_stream_read(buf, waves, sink, *, stream=None) -> None:
    """Reads the device buffer `buf` once (streaming-read probe,
    include/pkv_probe.h); sink: a device tensor of at least 256 bytes."""
    if not isinstance(buf, torch.Tensor) or not isinstance(sink, torch.Tensor):
        raise TypeError("buf and sink must be torch tensors")
    if sink.numel() * sink.element_size() < 256:
        raise ValueError("sink must hold at least 256 bytes")
    _same_device(buf, sink=sink)
    nbytes = buf.numel() * buf.element_size()
    _check("pkv_stream_read", _lib.pkv_stream_read(_ptr(buf), nbytes, int(waves), _ptr(sink),
                                                   _stream(stream)))
