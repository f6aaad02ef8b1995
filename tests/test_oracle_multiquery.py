"""Pins the oracle's multi-token write and causal multi-query attention.
CPU only.

Sequence b brings q_b new tokens, its last q_b positions (chunked prefill,
[B] "Continuous Batching"; verification of draft tokens in one pass, [A]
"How does speculative decoding interact with KV-cache compression"): row i
of the sequence is position p = T_b - q_b + i and attends over [0, p].

Each check is fixed by the pages or by mathematics, not by the oracle:
  * dense brute force: NumPy float64 causal attention on logical K/V that
    this file gathers itself, with the causal limit written out here;
  * one new token per sequence is the decode step: the write equals the
    single-token append byte for byte, the attention equals the decode
    attention;
  * identical keys with V[t] = t give the mean of 0..p = p / 2, which pins
    every row's position exactly;
  * a token changes only the rows at or after its position;
  * the write touches exactly the q_b slots of each sequence;
  * fp8: attention over decode(code) x scale, decoded by PyTorch.
"""
import math

import numpy as np
import pytest

from synthetic import (bf16_bits_from_f32, f32_from_bf16_bits, generate_multiquery,
                       make_workload)

TINY = "tiny_mq_b4_hq8_hkv2_d64_bs16"


def _written(orc, mq, g=0, **kw):
    base = mq.base
    kp, vp = base.k_pool[g].copy(), base.v_pool[g].copy()
    orc.write_tokens(mq.k_rows[g], mq.v_rows[g], mq.query_start, kp, vp, base.block_tables,
                     base.context_lens, mq.wl.block_size, **kw)
    return kp, vp


def _logical(pool, tables, T, bs):
    t = np.arange(T)
    return f32_from_bf16_bits(pool[tables[t // bs], t % bs]).astype(np.float64)


def _oracle(orc, mq, kp, vp, scale=None, layer=0, **kw):
    wl = mq.wl
    return orc.multiquery_attention(mq.query[layer], mq.query_start, kp, vp,
                                    mq.base.block_tables, mq.base.context_lens,
                                    mq.base.scale if scale is None else scale,
                                    block_size=wl.block_size, Hkv=wl.Hkv, **kw)


def _dense_causal(qrows, K, V, scale, G, T):
    """Rows [q, Hq, D] of one sequence; row i sees tokens 0 .. T - q + i."""
    nq, Hq, _ = qrows.shape
    out = np.zeros(qrows.shape)
    lse = np.zeros((nq, Hq))
    for i in range(nq):
        n = T - nq + i + 1
        for hq in range(Hq):
            s = scale * (K[:n, hq // G] @ qrows[i, hq])
            m = s.max()
            w = np.exp(s - m)
            out[i, hq] = (w[:, None] * V[:n, hq // G]).sum(0) / w.sum()
            lse[i, hq] = m + math.log(w.sum())
    return out, lse


@pytest.mark.parametrize("scale", [None, 1.0])
@pytest.mark.parametrize("seed", [0, 1])
def test_dense_causal_bruteforce(orc, scale, seed):
    mq = generate_multiquery(make_workload(TINY), seed=273010 + seed)
    wl = mq.wl
    kp, vp = _written(orc, mq)
    sc = float(mq.base.scale) if scale is None else scale
    out, lse = _oracle(orc, mq, kp, vp, scale=sc)
    q = f32_from_bf16_bits(mq.query[0]).astype(np.float64)
    assert mq.query_lens.max() > 1
    for b in range(wl.B):
        T = int(mq.base.context_lens[b])
        r0, r1 = int(mq.query_start[b]), int(mq.query_start[b + 1])
        K = _logical(kp, mq.base.block_tables[b], T, wl.block_size)
        V = _logical(vp, mq.base.block_tables[b], T, wl.block_size)
        ref, rl = _dense_causal(q[r0:r1], K, V, sc, wl.G, T)
        np.testing.assert_allclose(out[r0:r1], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[r0:r1], rl, rtol=0, atol=1e-12)


def test_whole_sequence_as_new_tokens(orc):
    """q_b = T_b: every token is new (a prefill chunk that starts at 0)."""
    wl = make_workload(TINY, ctx_fixed=(1, 5, 17, 40), max_blocks=3)
    mq = generate_multiquery(wl, query_lens=np.array([1, 5, 17, 40]))
    kp, vp = _written(orc, mq)
    assert not np.isnan(f32_from_bf16_bits(kp[mq.base.live > 0])[..., 0]).all()
    out, _ = _oracle(orc, mq, kp, vp, scale=1.0)
    q = f32_from_bf16_bits(mq.query[0]).astype(np.float64)
    for b in range(wl.B):
        T = int(mq.base.context_lens[b])
        r0, r1 = int(mq.query_start[b]), int(mq.query_start[b + 1])
        K = _logical(kp, mq.base.block_tables[b], T, wl.block_size)
        V = _logical(vp, mq.base.block_tables[b], T, wl.block_size)
        ref, _ = _dense_causal(q[r0:r1], K, V, 1.0, wl.G, T)
        np.testing.assert_allclose(out[r0:r1], ref, rtol=0, atol=1e-12)
        # the first row sees only token 0: exactly its V
        for hq in range(wl.Hq):
            assert np.array_equal(out[r0, hq], V[0, hq // wl.G])


def test_one_new_token_is_the_decode_step(orc):
    mq = generate_multiquery(make_workload(TINY), query_lens=np.ones(4, dtype=np.int32))
    wl, base = mq.wl, mq.base
    kp, vp = _written(orc, mq)
    ka, va = base.k_pool[0].copy(), base.v_pool[0].copy()
    orc.append(mq.k_rows[0], mq.v_rows[0], ka, va, base.block_tables, base.context_lens,
               wl.block_size)
    assert np.array_equal(kp, ka) and np.array_equal(vp, va)
    out, lse = _oracle(orc, mq, kp, vp)
    ref, rl = orc.paged_attention(mq.query[0], ka, va, base.block_tables, base.context_lens,
                                  base.scale, block_size=wl.block_size, Hkv=wl.Hkv)
    assert np.array_equal(out, ref) and np.array_equal(lse, rl)


def test_last_row_is_decode_over_the_whole_context(orc):
    mq = generate_multiquery(make_workload(TINY))
    wl, base = mq.wl, mq.base
    kp, vp = _written(orc, mq)
    out, lse = _oracle(orc, mq, kp, vp)
    last = mq.query_start[1:] - 1
    ref, rl = orc.paged_attention(np.ascontiguousarray(mq.query[0][last]), kp, vp,
                                  base.block_tables, base.context_lens, base.scale,
                                  block_size=wl.block_size, Hkv=wl.Hkv)
    assert np.array_equal(out[last], ref) and np.array_equal(lse[last], rl)


def test_identical_keys_pin_every_position(orc):
    """All keys equal and V[t] = t (exact in bf16 for t <= 256): row i of
    sequence b must give (T_b - q_b + i) / 2 in every element."""
    wl = make_workload(TINY, ctx_fixed=(3, 17, 100, 256), max_blocks=16)
    mq = generate_multiquery(wl, query_lens=np.array([3, 9, 5, 17]))
    base = mq.base
    kp, vp = _written(orc, mq)
    key = bf16_bits_from_f32(np.random.default_rng(5).standard_normal((wl.Hkv, wl.D)))
    kp[:, :] = key[None, None]
    for b in range(wl.B):
        for t in range(int(base.context_lens[b])):
            p = base.block_tables[b, t // wl.block_size]
            vp[p, t % wl.block_size] = bf16_bits_from_f32(np.full((wl.Hkv, wl.D), t, np.float32))
    out, _ = _oracle(orc, mq, kp, vp, scale=1.0)
    for b in range(wl.B):
        T, q = int(base.context_lens[b]), int(mq.query_lens[b])
        for i in range(q):
            p = T - q + i
            np.testing.assert_allclose(out[mq.query_start[b] + i], p / 2.0, rtol=0, atol=1e-12)


def test_a_token_changes_only_rows_at_or_after_it(orc):
    mq = generate_multiquery(make_workload(TINY), query_lens=np.array([1, 9, 3, 8]))
    wl, base = mq.wl, mq.base
    kp, vp = _written(orc, mq)
    out, _ = _oracle(orc, mq, kp, vp)
    b = 3
    T, q, r0 = int(base.context_lens[b]), int(mq.query_lens[b]), int(mq.query_start[b])
    for k in range(q):
        t = T - q + k                                   # position of new row k
        p = base.block_tables[b, t // wl.block_size]
        kp2, vp2 = kp.copy(), vp.copy()
        kp2[p, t % wl.block_size] = bf16_bits_from_f32(np.full((wl.Hkv, wl.D), 3.0, np.float32))
        vp2[p, t % wl.block_size] = bf16_bits_from_f32(np.full((wl.Hkv, wl.D), 50.0, np.float32))
        out2, _ = _oracle(orc, mq, kp2, vp2)
        for i in range(q):
            same = np.array_equal(out2[r0 + i], out[r0 + i])
            assert same == (i < k), (k, i)
        others = np.r_[0:r0, r0 + q:mq.rows]
        assert np.array_equal(out2[others], out[others])


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_write_touches_exactly_the_new_slots(orc, kv_dtype):
    mq = generate_multiquery(make_workload(TINY))
    wl, base = mq.wl, mq.base
    if kv_dtype == "bf16":
        src = (base.k_pool[0], base.v_pool[0])
        kw = {}
    else:
        ks = orc.fp8_block_scales(base.k_pool[0], base.block_tables, base.context_lens,
                                  wl.block_size)
        vs = orc.fp8_block_scales(base.v_pool[0], base.block_tables, base.context_lens,
                                  wl.block_size)
        src = (orc.fp8_quantize_pool(base.k_pool[0], ks), orc.fp8_quantize_pool(base.v_pool[0], vs))
        kw = dict(kv_dtype="fp8", k_scale=ks, v_scale=vs)
    kp, vp = src[0].copy(), src[1].copy()
    orc.write_tokens(mq.k_rows[0], mq.v_rows[0], mq.query_start, kp, vp, base.block_tables,
                     base.context_lens, wl.block_size, **kw)
    for before, rows, after, sc in ((src[0], mq.k_rows[0], kp, kw.get("k_scale")),
                                    (src[1], mq.v_rows[0], vp, kw.get("v_scale"))):
        changed = np.zeros(before.shape[:2], dtype=bool)
        for b in range(wl.B):
            T, q = int(base.context_lens[b]), int(mq.query_lens[b])
            for i in range(q):
                t = T - q + i
                p = int(base.block_tables[b, t // wl.block_size])
                row = rows[mq.query_start[b] + i]
                if kv_dtype == "bf16":
                    want = row
                else:
                    want = np.stack([orc.e4m3_quantize_array(row[h], float(sc[p, h]))
                                     for h in range(wl.Hkv)])
                assert np.array_equal(after[p, t % wl.block_size], want)
                changed[p, t % wl.block_size] = True
        assert np.array_equal(after[~changed], before[~changed])


def test_fp8_matches_dense_on_dequantised_values(orc):
    import torch

    wl = make_workload(TINY, kv_dtype="fp8")
    mq = generate_multiquery(wl)
    base = mq.base
    ks = orc.fp8_block_scales(base.k_pool[0], base.block_tables, base.context_lens,
                              wl.block_size)
    vs = orc.fp8_block_scales(base.v_pool[0], base.block_tables, base.context_lens,
                              wl.block_size)
    kc, vc = orc.fp8_quantize_pool(base.k_pool[0], ks), orc.fp8_quantize_pool(base.v_pool[0], vs)
    orc.write_tokens(mq.k_rows[0], mq.v_rows[0], mq.query_start, kc, vc, base.block_tables,
                     base.context_lens, wl.block_size, kv_dtype="fp8", k_scale=ks, v_scale=vs)
    out, lse = _oracle(orc, mq, kc, vc, kv_dtype="fp8", k_scale=ks, v_scale=vs)

    def deq(codes, sc):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return v * sc[:, None, :, None].astype(np.float64)

    kd, vd = deq(kc, ks), deq(vc, vs)
    q = f32_from_bf16_bits(mq.query[0]).astype(np.float64)
    for b in range(wl.B):
        T = int(base.context_lens[b])
        r0, r1 = int(mq.query_start[b]), int(mq.query_start[b + 1])
        t = np.arange(T)
        phys = base.block_tables[b][t // wl.block_size]
        K, V = kd[phys, t % wl.block_size], vd[phys, t % wl.block_size]
        ref, rl = _dense_causal(q[r0:r1], K, V, float(base.scale), wl.G, T)
        np.testing.assert_allclose(out[r0:r1], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[r0:r1], rl, rtol=0, atol=1e-12)


def test_more_new_tokens_than_context_is_rejected(orc):
    mq = generate_multiquery(make_workload(TINY))
    base = mq.base
    qs = mq.query_start.copy()
    qs[1:] += 1                          # sequence 0 (T = 1) now claims 2 tokens
    kp, vp = base.k_pool[0].copy(), base.v_pool[0].copy()
    rows = np.concatenate([mq.k_rows[0], mq.k_rows[0][:1]])
    with pytest.raises(ValueError):
        orc.write_tokens(rows, rows, qs, kp, vp, base.block_tables, base.context_lens,
                         mq.wl.block_size)
    q = np.concatenate([mq.query[0], mq.query[0][:1]])
    with pytest.raises(ValueError):
        orc.multiquery_attention(q, qs, kp, vp, base.block_tables, base.context_lens, 1.0,
                                 block_size=mq.wl.block_size, Hkv=mq.wl.Hkv)
