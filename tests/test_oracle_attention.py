"""Pins the oracle's paged attention, append and log-sum-exp merge.  CPU only.

Each check is fixed by the pages or by mathematics, not by the oracle:
  * dense brute force: NumPy float64 attention on logical (un-paged) K/V
    that this file gathers itself with fancy indexing;
  * one cached token gives exactly that token's V;
  * identical keys give the mean of V;
  * any permutation of physical placement ([B] "PagedAttention": any free
    block can hold any logical block) leaves the result bit-identical;
  * shared prefix blocks ([B] "PagedAttention", block sharing) equal private
    duplicated copies;
  * GQA equals MHA with repeated K/V heads ([B] "Attention Variants");
  * a needle key aligned with the query selects its V, at every slot;
  * NaN in holes and tail slots never reaches the output (only the last
    block of a sequence is partial);
  * split + merge equals the unsplit result.
"""
import math

import numpy as np
import pytest

from synthetic import (bf16_bits_from_f32, f32_from_bf16_bits, generate, make_workload,
                       random_partials)

TINY = "tiny_b4_hq8_hkv2_d64_bs16"


def _appended(orc, inp, g=0):
    """Host pools of group g after the decode step's append."""
    wl = inp.wl
    kp, vp = inp.k_pool[g].copy(), inp.v_pool[g].copy()
    orc.append(inp.k_new[g], inp.v_new[g], kp, vp, inp.block_tables, inp.context_lens,
               wl.block_size)
    return kp, vp


def _logical(pool, tables, T, bs):
    """[T, Hkv, D] float64 of one sequence, gathered with NumPy indexing."""
    t = np.arange(T)
    phys = tables[t // bs]
    return f32_from_bf16_bits(pool[phys, t % bs]).astype(np.float64)


def _dense(q, K, V, scale, G):
    """Textbook attention for one sequence: q [Hq, D], K/V [T, Hkv, D]."""
    Hq = q.shape[0]
    out = np.zeros((Hq, q.shape[1]))
    lse = np.zeros(Hq)
    for hq in range(Hq):
        k = K[:, hq // G, :]
        v = V[:, hq // G, :]
        s = scale * (k @ q[hq])
        m = s.max()
        w = np.exp(s - m)
        out[hq] = (w[:, None] * v).sum(0) / w.sum()
        lse[hq] = m + math.log(w.sum())
    return out, lse


def _oracle(orc, inp, kp, vp, scale=None, layer=0, **kw):
    wl = inp.wl
    return orc.paged_attention(inp.query[layer], kp, vp, inp.block_tables, inp.context_lens,
                               inp.scale if scale is None else scale,
                               block_size=wl.block_size, Hkv=wl.Hkv, **kw)


@pytest.mark.parametrize("scale", [None, 1.0])
def test_dense_bruteforce_tiny(orc, scale):
    inp = generate(make_workload(TINY))
    wl = inp.wl
    kp, vp = _appended(orc, inp)
    sc = float(inp.scale) if scale is None else scale
    out, lse = _oracle(orc, inp, kp, vp, scale=sc)
    q = f32_from_bf16_bits(inp.query[0]).astype(np.float64)
    for b in range(wl.B):
        T = int(inp.context_lens[b])
        K = _logical(kp, inp.block_tables[b], T, wl.block_size)
        V = _logical(vp, inp.block_tables[b], T, wl.block_size)
        ref, rlse = _dense(q[b], K, V, sc, wl.G)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], rlse, rtol=0, atol=1e-12)
        assert np.all(np.isfinite(out[b]))


def test_append_writes_only_the_new_slot(orc):
    inp = generate(make_workload(TINY))
    wl = inp.wl
    kp, vp = _appended(orc, inp)
    for src, new, dst in ((inp.k_pool[0], inp.k_new[0], kp), (inp.v_pool[0], inp.v_new[0], vp)):
        changed = np.zeros(src.shape[:2], dtype=bool)
        for b in range(wl.B):
            t = int(inp.context_lens[b]) - 1
            p = int(inp.block_tables[b, t // wl.block_size])
            assert np.array_equal(dst[p, t % wl.block_size], new[b])
            changed[p, t % wl.block_size] = True
        assert np.array_equal(dst[~changed], src[~changed])


def test_single_token_is_exactly_v(orc):
    wl = make_workload(TINY, ctx_fixed=(1, 1, 1, 1), max_blocks=2)
    inp = generate(wl)
    kp, vp = _appended(orc, inp)
    out, lse = _oracle(orc, inp, kp, vp)
    for b in range(wl.B):
        v = f32_from_bf16_bits(inp.v_new[0][b]).astype(np.float64)
        for hq in range(wl.Hq):
            assert np.array_equal(out[b, hq], v[hq // wl.G])


def test_identical_keys_give_mean_of_v(orc):
    inp = generate(make_workload(TINY))
    wl = inp.wl
    kp, vp = _appended(orc, inp)
    key = bf16_bits_from_f32(np.random.default_rng(3).standard_normal((wl.Hkv, wl.D)))
    kp[:, :] = key[None, None]
    out, _ = _oracle(orc, inp, kp, vp, scale=1.0)
    for b in range(wl.B):
        T = int(inp.context_lens[b])
        V = _logical(vp, inp.block_tables[b], T, wl.block_size)
        for hq in range(wl.Hq):
            np.testing.assert_allclose(out[b, hq], V[:, hq // wl.G].mean(0), rtol=0,
                                       atol=1e-12)


def _permute(inp, kp, vp, seed):
    rng = np.random.default_rng(seed)
    nb = kp.shape[0]
    perm = rng.permutation(nb)          # new position of old block i is perm[i]
    kq = np.empty_like(kp)
    vq = np.empty_like(vp)
    kq[perm] = kp
    vq[perm] = vp
    tables = np.where(inp.block_tables >= 0, perm[np.maximum(inp.block_tables, 0)], -1)
    return kq, vq, tables.astype(np.int32)


def test_physical_permutation_is_bit_identical(orc):
    inp = generate(make_workload(TINY))
    wl = inp.wl
    kp, vp = _appended(orc, inp)
    base, blse = _oracle(orc, inp, kp, vp)
    for seed in (1, 2, 3):
        kq, vq, tq = _permute(inp, kp, vp, seed)
        out, lse = orc.paged_attention(inp.query[0], kq, vq, tq, inp.context_lens, inp.scale,
                                       block_size=wl.block_size, Hkv=wl.Hkv)
        assert np.array_equal(out, base) and np.array_equal(lse, blse)


def test_shared_prefix_equals_private_copies(orc):
    wl = make_workload("llama70b_b4_ctx32k_split512_prefix2k", ctx_fixed=(100, 70, 64, 90),
                       shared_prefix_blocks=4, max_blocks=8, Hq=8, Hkv=2, D=64,
                       split_tokens=0)
    inp = generate(wl)
    kp, vp = _appended(orc, inp)
    shared, slse = _oracle(orc, inp, kp, vp)
    # give every sequence a private copy of the prefix blocks
    nb = kp.shape[0]
    extra = (wl.B - 1) * wl.shared_prefix_blocks
    kq = np.concatenate([kp, np.zeros((extra,) + kp.shape[1:], kp.dtype)])
    vq = np.concatenate([vp, np.zeros((extra,) + vp.shape[1:], vp.dtype)])
    tq = inp.block_tables.copy()
    nxt = nb
    for b in range(1, wl.B):
        for j in range(wl.shared_prefix_blocks):
            src = tq[b, j]
            kq[nxt] = kp[src]
            vq[nxt] = vp[src]
            tq[b, j] = nxt
            nxt += 1
    out, lse = orc.paged_attention(inp.query[0], kq, vq, tq, inp.context_lens, inp.scale,
                                   block_size=wl.block_size, Hkv=wl.Hkv)
    assert np.array_equal(out, shared) and np.array_equal(lse, slse)
    assert len(set(tq[:, 0])) == wl.B and len(set(inp.block_tables[:, 0])) == 1


@pytest.mark.parametrize("Hkv", [1, 2, 8])   # MQA, GQA, MHA
def test_gqa_equals_mha_with_repeated_heads(orc, Hkv):
    wl = make_workload(TINY, Hkv=Hkv)
    inp = generate(wl)
    kp, vp = _appended(orc, inp)
    out, lse = _oracle(orc, inp, kp, vp)
    G = wl.G
    kr = np.ascontiguousarray(np.repeat(kp, G, axis=2))
    vr = np.ascontiguousarray(np.repeat(vp, G, axis=2))
    out2, lse2 = orc.paged_attention(inp.query[0], kr, vr, inp.block_tables, inp.context_lens,
                                     inp.scale, block_size=wl.block_size, Hkv=wl.Hq)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_needle_at_every_slot(orc):
    """A key equal to 64 x the (shared) query dominates the softmax: the
    output is that token's V.  Swept over every slot of every block,
    including the partial last block."""
    wl = make_workload(TINY, ctx_fixed=(100, 37, 16, 5), max_blocks=7)
    inp = generate(wl)
    kp, vp = _appended(orc, inp)
    q = inp.query[0].copy()
    for b in range(wl.B):
        for h in range(wl.Hkv):
            q[b, h * wl.G:(h + 1) * wl.G] = q[b, h * wl.G]   # one query per group
    qf = f32_from_bf16_bits(q).astype(np.float64)
    for b in range(wl.B):
        T = int(inp.context_lens[b])
        for p in range(T):
            kk = kp.copy()
            phys = int(inp.block_tables[b, p // wl.block_size])
            for h in range(wl.Hkv):
                kk[phys, p % wl.block_size, h] = bf16_bits_from_f32(
                    (64.0 * qf[b, h * wl.G] * math.sqrt(wl.D) * 8).astype(np.float32))
            out, _ = orc.paged_attention(q, kk, vp, inp.block_tables, inp.context_lens, 1.0,
                                         block_size=wl.block_size, Hkv=wl.Hkv)
            want = f32_from_bf16_bits(vp[phys, p % wl.block_size]).astype(np.float64)
            for hq in range(wl.Hq):
                np.testing.assert_allclose(out[b, hq], want[hq // wl.G], atol=1e-9, rtol=0)


def test_poison_never_reaches_output(orc):
    inp = generate(make_workload(TINY))
    wl = inp.wl
    kp, vp = _appended(orc, inp)
    out, lse = _oracle(orc, inp, kp, vp)
    assert np.all(np.isfinite(out))
    # zeroing every dead slot instead of NaN changes nothing
    dead = np.arange(wl.block_size)[None, :] >= inp.live[:, None]
    assert dead.sum() > 0
    kz, vz = kp.copy(), vp.copy()
    kz[dead] = 0
    vz[dead] = 0
    out2, lse2 = _oracle(orc, inp, kz, vz)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_missing_append_is_visible(orc):
    """Before the append, the new token's slot holds NaN and poisons the result."""
    inp = generate(make_workload(TINY))
    out, _ = _oracle(orc, inp, inp.k_pool[0], inp.v_pool[0])
    assert np.all(np.isnan(out))


@pytest.mark.parametrize("S", [16, 48, 512, 1024])
def test_split_then_merge_equals_unsplit(orc, S):
    inp = generate(make_workload(TINY))
    wl = inp.wl
    kp, vp = _appended(orc, inp)
    base, blse = _oracle(orc, inp, kp, vp)
    ms = (int(inp.context_lens.max()) + S - 1) // S
    out, lse, po, pl = _oracle(orc, inp, kp, vp, split_tokens=S, max_splits=ms,
                               want_partials=True)
    np.testing.assert_allclose(out, base, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)
    # each partial is the plain attention over its own token range
    q = f32_from_bf16_bits(inp.query[0]).astype(np.float64)
    for b in range(wl.B):
        T = int(inp.context_lens[b])
        K = _logical(kp, inp.block_tables[b], T, wl.block_size)
        V = _logical(vp, inp.block_tables[b], T, wl.block_size)
        for s in range(ms):
            if s * S >= T:
                assert np.all(np.isnan(pl[b, :, s]))
                continue
            r, rl = _dense(q[b], K[s * S:(s + 1) * S], V[s * S:(s + 1) * S], float(inp.scale),
                           wl.G)
            np.testing.assert_allclose(po[b, :, s], r, rtol=0, atol=1e-12)
            np.testing.assert_allclose(pl[b, :, s], rl, rtol=0, atol=1e-12)


def test_merge_single_part_is_identity(orc):
    rng = np.random.default_rng(5)
    o = rng.standard_normal((1, 64))
    out, lse = orc.lse_merge(o, np.array([0.37]))
    assert np.array_equal(out, o[0]) and lse == 0.37


def test_merge_ignores_empty_parts(orc):
    rng = np.random.default_rng(6)
    o = rng.standard_normal((4, 32))
    l = np.array([0.5, -np.inf, 2.0, -np.inf])
    o[1] = 0
    o[3] = 0
    out, lse = orc.lse_merge(o, l)
    out2, lse2 = orc.lse_merge(o[[0, 2]], l[[0, 2]])
    assert np.array_equal(out, out2) and lse == lse2
    out3, lse3 = orc.lse_merge(np.zeros((2, 32)), np.array([-np.inf, -np.inf]))
    assert lse3 == -np.inf and np.all(out3 == 0)


def test_merge_matches_closed_form(orc):
    """Two parts over disjoint keys: merged lse = log(e^a + e^b) and the output
    is the e^lse-weighted mix."""
    rng = np.random.default_rng(8)
    o = rng.standard_normal((2, 16))
    a, b = 1.3, -0.4
    out, lse = orc.lse_merge(o, np.array([a, b]))
    assert abs(lse - math.log(math.exp(a) + math.exp(b))) < 1e-14
    wa = math.exp(a) / (math.exp(a) + math.exp(b))
    np.testing.assert_allclose(out, wa * o[0] + (1 - wa) * o[1], atol=1e-14, rtol=0)


def test_split_reduce_layout(orc):
    """orc_split_reduce reads [B, Hq, max_splits, D] partials and only the
    ceil(T/S) live splits of each sequence (the rest are NaN)."""
    ctx = np.array([1, 17, 100, 513], dtype=np.int32)
    S, Hq, D = 32, 4, 8
    ms = 17
    po, pl = random_partials(11, ctx, Hq, D, S, ms, empty_fraction=0.2)
    out, lse = orc.split_reduce(po, pl, ctx, S)
    for b in range(4):
        ns = (ctx[b] + S - 1) // S
        for h in range(Hq):
            r, rl = orc.lse_merge(po[b, h, :ns].astype(np.float64), pl[b, h, :ns].astype(np.float64))
            assert np.array_equal(out[b, h], r) and (lse[b, h] == rl or (np.isinf(rl) and np.isinf(lse[b, h])))
    assert np.all(np.isfinite(out))


def test_fp8_attention_matches_dense_on_dequantised_values(orc):
    """The fp8 path attends over decode(code) x scale ([B] "FP8 KV cache":
    dequantise on read); the dequantisation here uses PyTorch's decoder."""
    import torch

    wl = make_workload("fp8_36layers_groups4_b32_ctx2k_8k", B=3, ctx_uniform=(20, 90),
                       max_blocks=8, layers=4, Hq=8, Hkv=2, D=64)
    inp = generate(wl)
    src_k, src_v = inp.k_pool[0], inp.v_pool[0]
    ks = orc.fp8_block_scales(src_k, inp.block_tables, inp.context_lens, wl.block_size)
    vs = orc.fp8_block_scales(src_v, inp.block_tables, inp.context_lens, wl.block_size)
    kc, vc = orc.fp8_quantize_pool(src_k, ks), orc.fp8_quantize_pool(src_v, vs)
    orc.append(inp.k_new[0], inp.v_new[0], kc, vc, inp.block_tables, inp.context_lens,
               wl.block_size, kv_dtype="fp8", k_scale=ks, v_scale=vs)
    out, lse = orc.paged_attention(inp.query[0], kc, vc, inp.block_tables, inp.context_lens,
                                   inp.scale, block_size=wl.block_size, Hkv=wl.Hkv,
                                   kv_dtype="fp8", k_scale=ks, v_scale=vs)

    def deq(codes, sc):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return v * sc[:, None, :, None].astype(np.float64)

    kd, vd = deq(kc, ks), deq(vc, vs)
    q = f32_from_bf16_bits(inp.query[0]).astype(np.float64)
    for b in range(wl.B):
        T = int(inp.context_lens[b])
        t = np.arange(T)
        phys = inp.block_tables[b][t // wl.block_size]
        K, V = kd[phys, t % wl.block_size], vd[phys, t % wl.block_size]
        ref, rl = _dense(q[b], K, V, float(inp.scale), wl.G)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl, rtol=0, atol=1e-12)
