"""Helpers for the GPU parity tests: upload seeded host inputs, run the HIP
path through the C ABI binding, compare with the CPU oracle.

Tolerance for attention outputs (fp32 accumulate from bf16 / dequantised
fp8 inputs): elementwise |gpu - oracle| <= 2e-3 + 1e-2 * |oracle|.
Append and indexing results are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

ATOL = 2e-3
RTOL = 1e-2


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def tables_to_dev(block_tables, context_lens, block_size, num_blocks):
    """Device copies of a block table and its context lengths, after the
    oracle's validator has checked the preconditions every kernel relies
    on (live entries inside the pool, every sequence fits its row)."""
    import oracle

    st = oracle.check_tables(block_tables, context_lens, block_size, num_blocks)
    assert st == 0, f"invalid block table: sequence {-st - 1} breaks the preconditions"
    return to_dev(block_tables), to_dev(context_lens)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def assert_close(gpu, ref, what=""):
    g = gpu.detach().cpu().numpy().astype(np.float64) if isinstance(gpu, torch.Tensor) else gpu
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (ATOL + RTOL * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of "
                             f"tolerance; worst at {i}: gpu {g[i]!r} oracle {ref[i]!r}")
    return float(err.max())


class DeviceInputs:
    """Device copies of one workload's arrays (one cache group)."""

    def __init__(self, inp, group=0, k_pool=None, v_pool=None, k_scale=None, v_scale=None):
        self.inp = inp
        kp = inp.k_pool[group] if k_pool is None else k_pool
        vp = inp.v_pool[group] if v_pool is None else v_pool
        self.k = to_dev(kp)
        self.v = to_dev(vp)
        self.k_new = to_dev(inp.k_new[group])
        self.v_new = to_dev(inp.v_new[group])
        self.q = to_dev(inp.query)
        self.bt, self.cl = tables_to_dev(inp.block_tables, inp.context_lens,
                                         inp.wl.block_size, kp.shape[0])
        self.ks = None if k_scale is None else to_dev(k_scale)
        self.vs = None if v_scale is None else to_dev(v_scale)


def run_step(pkv, d: DeviceInputs, layer=0, split_tokens=0, scale=None, append=True,
             want_lse=False, kv_dtype=None):
    """append (optional) + attention (+ reduce when split).  Returns out, lse.
    kv_dtype: the cache format name (default: inferred from the cache dtype)."""
    inp = d.inp
    wl = inp.wl
    sc = float(inp.scale) if scale is None else float(scale)
    fmt = None if kv_dtype in (None, "bf16", "fp8") else kv_dtype
    if append:
        pkv.paged_kv_append(d.k_new, d.v_new, d.k, d.v, d.bt, d.cl, k_scale=d.ks,
                            v_scale=d.vs, kv_dtype=fmt)
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device=dev()) if want_lse else None
    if split_tokens == 0:
        out = pkv.paged_decode_attention(d.q[layer], d.k, d.v, d.bt, d.cl, sc, lse_out=lse,
                                         k_scale=d.ks, v_scale=d.vs, kv_dtype=fmt)
    else:
        ms = pkv.max_splits_for(int(inp.context_lens.max()), split_tokens)
        po = torch.full((wl.B, wl.Hq, ms, wl.D), float("nan"), device=dev())
        pl = torch.full((wl.B, wl.Hq, ms), float("nan"), device=dev())
        pkv.paged_decode_attention(d.q[layer], d.k, d.v, d.bt, d.cl, sc,
                                   split_tokens=split_tokens, partial_out=po, partial_lse=pl,
                                   k_scale=d.ks, v_scale=d.vs, kv_dtype=fmt)
        out = pkv.split_context_reduce(po, pl, d.cl, split_tokens, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def host_appended(orc, inp, group=0, kv_dtype="bf16", k_pool=None, v_pool=None, ks=None,
                  vs=None):
    kp = (inp.k_pool[group] if k_pool is None else k_pool).copy()
    vp = (inp.v_pool[group] if v_pool is None else v_pool).copy()
    orc.append(inp.k_new[group], inp.v_new[group], kp, vp, inp.block_tables, inp.context_lens,
               inp.wl.block_size, kv_dtype=kv_dtype, k_scale=ks, v_scale=vs)
    return kp, vp


def fp8_group(orc, inp, group=0):
    """E4M3FN codes + per-(block, head) scales of one group, built by the
    oracle's encoder from the group's bf16 source values."""
    wl = inp.wl
    ks = orc.fp8_block_scales(inp.k_pool[group], inp.block_tables, inp.context_lens,
                              wl.block_size)
    vs = orc.fp8_block_scales(inp.v_pool[group], inp.block_tables, inp.context_lens,
                              wl.block_size)
    return orc.fp8_quantize_pool(inp.k_pool[group], ks), orc.fp8_quantize_pool(
        inp.v_pool[group], vs), ks, vs


def sample_rows(B, Hq, n, seed=0):
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (B - 1, Hq - 1)}
    while len(rows) < min(n, B * Hq):
        rows.add((int(rng.integers(B)), int(rng.integers(Hq))))
    return sorted(rows)


def host_threads():
    """Host threads for the oracle (this process's CPU affinity, at most 16)."""
    import os

    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_rows(orc, query, kp, vp, tables, lens, scale, *, block_size, Hkv, kv_dtype="bf16",
                ks=None, vs=None, rows=None):
    """Oracle output and lse of every (sequence, query head) row (or of the
    listed rows), one row per task on a pool of host threads (the oracle's
    ctypes calls release the GIL).  Returns out [n, D], lse [n] in row order
    and the row list."""
    import concurrent.futures as cf

    B, Hq, D = query.shape
    if rows is None:
        rows = [(b, hq) for b in range(B) for hq in range(Hq)]

    def one(r):
        b, hq = r
        return orc.attend_range(query, kp, vp, tables, b, hq, 0, int(lens[b]), scale,
                                block_size=block_size, Hkv=Hkv, kv_dtype=kv_dtype,
                                k_scale=ks, v_scale=vs)

    with cf.ThreadPoolExecutor(host_threads()) as ex:
        res = list(ex.map(one, rows, chunksize=8))
    return np.stack([o for o, _ in res]), np.array([l for _, l in res]), rows
