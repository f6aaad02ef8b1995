"""Seeded synthetic paged-KV workloads.

Shapes, value distributions and table structure follow the decode
workloads this library is measured on (model shapes from the pages'
worked examples: the Llama-3.1-8B shape of 32 query / 8 KV heads with
head_dim 128, the 70B shape of 64 query / 8 KV heads; block sizes 16 and
32 from [B] "PagedAttention"; cross-layer groups of 4 over 36 layers from
[A] "What is cross-layer KV sharing").

Pages: [A] "KV-Cache Engineering: Paged Attention, Prefix Cache,
Disaggregation (2026)"; [B] "KV Cache Engineering: PagedAttention,
Continuous Batching, Attention Variants, and the Bandwidth Wall".

Recipe (the same for every workload):
  * RNG: NumPy PCG64 streams keyed by (seed, stream id, chunk index), so
    the arrays do not depend on the thread count used to fill them.
  * K, V: N(0, 1) binary32 draws rounded to bf16 (nearest-even).
  * query: N(0, 1) / sqrt(D) rounded to bf16.
  * Physical placement: a seeded permutation of the pool; logical block j
    of sequence b takes the next unused entry of that permutation, so the
    blocks of one sequence are scattered and interleaved with holes.
  * Poison: every element of a block no table references (a hole), every
    slot past a sequence's last token, and the slot the decode step's
    append will write (position T - 1) hold a bf16 quiet NaN (0x7FC0).
    A kernel that reads any of them before the append, or ever reads a
    hole or tail slot, produces NaN.
  * Appended token: k_new, v_new [B, Hkv, D], fresh N(0, 1) bf16 draws.

Several new tokens per sequence (generate_multiquery): sequence b brings
q_b new tokens, the last q_b of its T_b (chunked prefill, [B] "Continuous
Batching"; the target's verification of draft tokens, [A] "How does
speculative decoding interact with KV-cache compression").  q_b is drawn
uniformly from the workload's q range and clipped to T_b; the q_b write
slots hold NaN before the write; K/V rows [rows, Hkv, D] and query rows
[layers, rows, Hq, D] are fresh draws with the same distributions.

Nothing here computes attention, quantises, or merges; the fp8 workload
carries bf16 source values, and each consumer quantises them with its own
encoder.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

BF16_QNAN = 0x7FC0
_CHUNK = 1 << 22

# stream ids
_S_CTX, _S_PERM, _S_K, _S_V, _S_Q, _S_KNEW, _S_VNEW, _S_PART = range(1, 9)
_S_QLEN, _S_KROWS, _S_VROWS, _S_QROWS = range(9, 13)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> binary32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_bf16(key: Tuple[int, ...], n: int, sigma: float = 1.0) -> np.ndarray:
    """n bf16 draws of N(0, sigma^2), filled chunk by chunk in parallel."""
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        rng = np.random.default_rng(list(key) + [c])
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[lo:hi] = bf16_bits_from_f32(x)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


@dataclass(frozen=True)
class Workload:
    """One decode-attention workload: shapes, context mix, pool structure."""

    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    max_blocks: int
    kv_dtype: str = "bf16"            # "bf16" or "fp8" (E4M3FN codes + scales)
    ctx_fixed: Tuple[int, ...] = ()   # explicit per-sequence lengths, or
    ctx_uniform: Tuple[int, int] = (0, 0)  # integers uniform in [lo, hi]
    pool: str = "exact"               # "exact" | "holes10" | "fixed:<n>"
    shared_prefix_blocks: int = 0     # logical blocks 0..n-1 shared by all
    split_tokens: int = 0             # 0: single pass
    layers: int = 1                   # logical layers per decode step
    layers_per_group: int = 1         # consecutive layers sharing one cache
    q_uniform: Tuple[int, int] = (1, 1)  # new tokens per sequence (multi-query)
    seed: int = 273000

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def groups(self) -> int:
        return self.layers // self.layers_per_group

    @property
    def bytes_per_elem(self) -> int:
        return 1 if self.kv_dtype == "fp8" else 2


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        # tiny oracle-sized case: 4 ragged sequences in a 64-block pool
        Workload("tiny_b4_hq8_hkv2_d64_bs16", B=4, Hq=8, Hkv=2, D=64, block_size=16,
                 max_blocks=33, ctx_fixed=(1, 17, 100, 513), pool="fixed:64",
                 seed=273000),
        # Llama-3.1-8B single-layer shape, 32 x 4096 tokens, pool sized exactly
        Workload("llama8b_b32_ctx4096_bs16", B=32, Hq=32, Hkv=8, D=128, block_size=16,
                 max_blocks=256, ctx_fixed=(4096,) * 32, pool="exact", seed=273001),
        # Llama-3.1-70B single-layer shape, 64 ragged sequences, 10% free holes
        Workload("llama70b_b64_ragged1k_16k_bs32", B=64, Hq=64, Hkv=8, D=128,
                 block_size=32, max_blocks=512, ctx_uniform=(1024, 16384),
                 pool="holes10", seed=273002),
        # long context, 512-token splits, 2048-token prefix shared by 4 tables
        Workload("llama70b_b4_ctx32k_split512_prefix2k", B=4, Hq=64, Hkv=8, D=128,
                 block_size=16, max_blocks=2048, ctx_fixed=(32768,) * 4, pool="exact",
                 shared_prefix_blocks=128, split_tokens=512, seed=273003),
        # several new tokens per sequence: ragged 1..17 (tiny, oracle-sized)
        Workload("tiny_mq_b4_hq8_hkv2_d64_bs16", B=4, Hq=8, Hkv=2, D=64, block_size=16,
                 max_blocks=33, ctx_fixed=(1, 17, 100, 513), pool="fixed:64",
                 q_uniform=(1, 17), seed=273010),
        # verification of 4 draft tokens per sequence on the 70B ragged batch
        Workload("llama70b_b64_ragged1k_16k_bs32_verify4", B=64, Hq=64, Hkv=8, D=128,
                 block_size=32, max_blocks=512, ctx_uniform=(1024, 16384),
                 pool="holes10", q_uniform=(4, 4), seed=273002),
        # chunked prefill: the last 512 tokens of 4 x 8192-token prompts are new
        Workload("llama8b_b4_ctx8k_chunk512", B=4, Hq=32, Hkv=8, D=128, block_size=16,
                 max_blocks=512, ctx_fixed=(8192,) * 4, pool="exact", q_uniform=(512, 512),
                 seed=273005),
        # fp8 cache, 36 layers in 9 groups of 4 sharing one cache per group
        Workload("fp8_36layers_groups4_b32_ctx2k_8k", B=32, Hq=32, Hkv=4, D=128,
                 block_size=16, max_blocks=512, kv_dtype="fp8",
                 ctx_uniform=(2048, 8192), pool="exact", layers=36,
                 layers_per_group=4, seed=273004),
    ]
}


def make_workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (smaller tests)."""
    import dataclasses

    return dataclasses.replace(WORKLOADS[name], **overrides)


@dataclass
class PagedInputs:
    """Host arrays of one workload (all numpy, C-contiguous)."""

    wl: Workload
    context_lens: np.ndarray           # [B] int32, includes the appended token
    block_tables: np.ndarray           # [B, max_blocks] int32, -1 past the end
    num_blocks: int
    live: np.ndarray                   # [num_blocks] int32 live slots per block
    k_pool: List[np.ndarray]           # per group [nb, bs, Hkv, D] bf16 bits
    v_pool: List[np.ndarray]
    k_new: List[np.ndarray]            # per group [B, Hkv, D] bf16 bits
    v_new: List[np.ndarray]
    query: np.ndarray                  # [layers, B, Hq, D] bf16 bits
    scale: np.float32 = field(default_factory=lambda: np.float32(0))

    @property
    def max_splits(self) -> int:
        S = self.wl.split_tokens
        if S <= 0:
            return 0
        return int(max(1, (int(self.context_lens.max()) + S - 1) // S))


def _context_lens(wl: Workload, seed: int) -> np.ndarray:
    if wl.ctx_fixed:
        assert len(wl.ctx_fixed) == wl.B
        return np.asarray(wl.ctx_fixed, dtype=np.int32)
    lo, hi = wl.ctx_uniform
    rng = np.random.default_rng([seed, _S_CTX])
    return rng.integers(lo, hi, size=wl.B, endpoint=True).astype(np.int32)


def _tables(wl: Workload, ctx: np.ndarray, seed: int):
    bs = wl.block_size
    nblk = (ctx.astype(np.int64) + bs - 1) // bs
    assert int(nblk.max()) <= wl.max_blocks, "context exceeds table width"
    shared = wl.shared_prefix_blocks
    needed = int(nblk.sum()) - shared * (wl.B - 1) if shared else int(nblk.sum())
    if wl.pool == "exact":
        num_blocks = needed
    elif wl.pool == "holes10":
        num_blocks = int(math.ceil(needed / 0.9))
    elif wl.pool.startswith("fixed:"):
        num_blocks = int(wl.pool.split(":")[1])
        assert num_blocks >= needed
    else:
        raise ValueError(wl.pool)
    rng = np.random.default_rng([seed, _S_PERM])
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((wl.B, wl.max_blocks), -1, dtype=np.int32)
    cursor = 0
    if shared:
        assert int(nblk.min()) >= shared
        prefix = perm[:shared]
        cursor = shared
        tables[:, :shared] = prefix[None, :]
    for b in range(wl.B):
        start = shared if shared else 0
        n = int(nblk[b]) - start
        tables[b, start:start + n] = perm[cursor:cursor + n]
        cursor += n
    assert cursor == needed
    live = np.zeros(num_blocks, dtype=np.int32)
    for b in range(wl.B):
        T = int(ctx[b])
        for j in range(int(nblk[b])):
            p = tables[b, j]
            live[p] = max(live[p], min(bs, T - j * bs))
    return tables, num_blocks, live


def _poison(pool: np.ndarray, live: np.ndarray, ctx: np.ndarray, tables: np.ndarray,
            bs: int) -> None:
    """NaN into holes, tail slots and every sequence's append slot (T - 1)."""
    nb = pool.shape[0]
    slot_idx = np.arange(bs, dtype=np.int32)[None, :]
    dead = slot_idx >= live[:, None]                      # [nb, bs]
    pool[dead] = BF16_QNAN
    for b in range(ctx.shape[0]):
        T = int(ctx[b])
        if T <= 0:
            continue
        t = T - 1
        p = int(tables[b, t // bs])
        pool[p, t % bs] = BF16_QNAN
    assert pool.shape[0] == nb


def generate(wl: Workload, seed: Optional[int] = None,
             groups: Optional[List[int]] = None) -> PagedInputs:
    """Draws the host arrays of `wl` (deterministic in `seed`).

    groups: which cache groups to materialise (default: all).  Tables,
    lengths and queries are always drawn in full.
    """
    seed = wl.seed if seed is None else int(seed)
    ctx = _context_lens(wl, seed)
    tables, num_blocks, live = _tables(wl, ctx, seed)
    bs, Hkv, D = wl.block_size, wl.Hkv, wl.D
    n_pool = num_blocks * bs * Hkv * D
    groups = list(range(wl.groups)) if groups is None else list(groups)
    k_pool, v_pool, k_new, v_new = [], [], [], []
    for g in groups:
        kp = _normal_bf16((seed, _S_K, g), n_pool).reshape(num_blocks, bs, Hkv, D)
        vp = _normal_bf16((seed, _S_V, g), n_pool).reshape(num_blocks, bs, Hkv, D)
        _poison(kp, live, ctx, tables, bs)
        _poison(vp, live, ctx, tables, bs)
        k_pool.append(kp)
        v_pool.append(vp)
        k_new.append(_normal_bf16((seed, _S_KNEW, g), wl.B * Hkv * D).reshape(wl.B, Hkv, D))
        v_new.append(_normal_bf16((seed, _S_VNEW, g), wl.B * Hkv * D).reshape(wl.B, Hkv, D))
    query = _normal_bf16((seed, _S_Q), wl.layers * wl.B * wl.Hq * D,
                         sigma=1.0 / math.sqrt(D)).reshape(wl.layers, wl.B, wl.Hq, D)
    return PagedInputs(wl=wl, context_lens=ctx, block_tables=tables, num_blocks=num_blocks,
                       live=live, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new,
                       query=query, scale=np.float32(1.0 / math.sqrt(D)))


@dataclass
class MultiQueryInputs:
    """Host arrays of a multi-query step (all numpy, C-contiguous)."""

    base: PagedInputs                  # lengths, tables, pools (write slots poisoned)
    query_lens: np.ndarray             # [B] int32, 0 <= q_b <= T_b
    query_start: np.ndarray            # [B + 1] int32, prefix sums of query_lens
    k_rows: List[np.ndarray]           # per group [rows, Hkv, D] bf16 bits
    v_rows: List[np.ndarray]
    query: np.ndarray                  # [layers, rows, Hq, D] bf16 bits

    @property
    def wl(self) -> Workload:
        return self.base.wl

    @property
    def rows(self) -> int:
        return int(self.query_start[-1])


def generate_multiquery(wl: Workload, seed: Optional[int] = None,
                        groups: Optional[List[int]] = None,
                        query_lens: Optional[np.ndarray] = None) -> MultiQueryInputs:
    """Draws a step in which sequence b writes and attends q_b new tokens.

    query_lens overrides the drawn q_b (each clipped to [0, T_b])."""
    seed = wl.seed if seed is None else int(seed)
    base = generate(wl, seed, groups)
    ctx = base.context_lens
    if query_lens is None:
        lo, hi = wl.q_uniform
        rng = np.random.default_rng([seed, _S_QLEN])
        q = rng.integers(lo, hi, size=wl.B, endpoint=True)
    else:
        q = np.asarray(query_lens, dtype=np.int64)
    q = np.clip(q, 0, ctx).astype(np.int32)
    qs = np.zeros(wl.B + 1, dtype=np.int32)
    qs[1:] = np.cumsum(q)
    rows = int(qs[-1])
    bs = wl.block_size
    for pool in base.k_pool + base.v_pool:
        for b in range(wl.B):
            for t in range(int(ctx[b]) - int(q[b]), int(ctx[b])):
                pool[int(base.block_tables[b, t // bs]), t % bs] = BF16_QNAN
    groups = list(range(wl.groups)) if groups is None else list(groups)
    n = rows * wl.Hkv * wl.D
    k_rows = [_normal_bf16((seed, _S_KROWS, g), n).reshape(rows, wl.Hkv, wl.D) for g in groups]
    v_rows = [_normal_bf16((seed, _S_VROWS, g), n).reshape(rows, wl.Hkv, wl.D) for g in groups]
    query = _normal_bf16((seed, _S_QROWS), wl.layers * rows * wl.Hq * wl.D,
                         sigma=1.0 / math.sqrt(wl.D)).reshape(wl.layers, rows, wl.Hq, wl.D)
    return MultiQueryInputs(base=base, query_lens=q, query_start=qs, k_rows=k_rows,
                            v_rows=v_rows, query=query)


def random_partials(seed: int, context_lens: np.ndarray, Hq: int, D: int,
                    split_tokens: int, max_splits: int, empty_fraction: float = 0.0):
    """Random split partials for exercising a log-sum-exp reduction alone.

    partial_out [B, Hq, max_splits, D] ~ N(0, 1); partial_lse ~ N(0, 4)
    for the ceil(T / split_tokens) live splits of each sequence, NaN in
    every slot past them.  `empty_fraction` of the live splits get
    lse = -inf and out = 0 (the representation of a split with no tokens).
    """
    B = context_lens.shape[0]
    rng = np.random.default_rng([seed, _S_PART])
    po = rng.standard_normal((B, Hq, max_splits, D), dtype=np.float32)
    pl = (rng.standard_normal((B, Hq, max_splits), dtype=np.float32) * np.float32(2.0))
    ns = (context_lens.astype(np.int64) + split_tokens - 1) // split_tokens
    s_idx = np.arange(max_splits)[None, None, :]
    dead = s_idx >= ns[:, None, None]
    po[np.broadcast_to(dead[..., None], po.shape)] = np.nan
    pl[np.broadcast_to(dead, pl.shape)] = np.nan
    if empty_fraction > 0:
        emp = (rng.random(pl.shape) < empty_fraction) & ~dead
        pl[emp] = -np.inf
        po[np.broadcast_to(emp[..., None], po.shape)] = 0.0
    return po, pl
