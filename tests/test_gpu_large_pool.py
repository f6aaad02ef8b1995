"""Pools larger than 4 GiB: every block a sequence uses sits past byte 2^32
of its pool, so a block offset computed in 32 bits anywhere on the path
(append, attention in every schedule, the split reduce, whole-block moves)
would read or write the wrong place.

The oracle gets the same blocks in a compact pool with the table remapped
to it; the result does not depend on where the blocks sit ([B]
"PagedAttention": the table is the only link between logical and physical
blocks), so the oracle on the compact layout is the reference.  The
appended rows and every used block are compared bit for bit; attention
outputs within the tolerance of the other parity tests.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, dev, tables_to_dev, to_dev
from synthetic import bf16_bits_from_f32

pytestmark = pytest.mark.gpu

B, HQ, HKV, D, BS = 4, 16, 8, 128, 32
CTX = np.array([1, 100, 1000, 3000], np.int32)     # one tile, ragged tails, many tiles
NAN_BF16 = np.uint16(0x7FC0)
NAN_E4M3 = np.uint8(0x7F)


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_273_amd as m

    return m


def _inputs(num_blocks, block_bytes, seed):
    """Compact host pools + tables, and the pool ids past 4 GiB the same
    blocks take on the device."""
    rng = np.random.default_rng(seed)
    nblk = (CTX + BS - 1) // BS
    total = int(nblk.sum())
    lowest = (1 << 32) // block_bytes + 1              # first id whose offset is past 2^32
    assert lowest + total <= num_blocks
    big = rng.choice(np.arange(lowest, num_blocks), size=total, replace=False).astype(np.int32)
    compact = np.full((B, int(nblk.max())), -1, np.int32)
    far = np.full_like(compact, -1)
    j = 0
    for b in range(B):
        for i in range(nblk[b]):
            compact[b, i], far[b, i] = j, big[j]
            j += 1

    def pool():
        x = bf16_bits_from_f32(rng.standard_normal((total, BS, HKV, D), dtype=np.float32))
        for b in range(B):                             # tail slots and the append slot: NaN
            for t in range(CTX[b] - 1, nblk[b] * BS):
                x[compact[b, t // BS], t % BS] = NAN_BF16
        return x

    k, v = pool(), pool()
    q = bf16_bits_from_f32(rng.standard_normal((B, HQ, D), dtype=np.float32) / np.sqrt(D))
    kn = bf16_bits_from_f32(rng.standard_normal((B, HKV, D), dtype=np.float32))
    vn = bf16_bits_from_f32(rng.standard_normal((B, HKV, D), dtype=np.float32))
    return dict(k=k, v=v, q=q, kn=kn, vn=vn, compact=compact, far=far, big=big, total=total)


def _device_pool(host_blocks, big, num_blocks, dtype):
    """A device pool of num_blocks whose blocks `big` hold host_blocks (the
    rest is never read)."""
    pool = torch.empty((num_blocks,) + host_blocks.shape[1:], dtype=dtype, device=dev())
    pool[torch.from_numpy(big.astype(np.int64)).to(dev())] = to_dev(host_blocks).view(dtype)
    return pool


def _blocks(pool, big):
    return pool[torch.from_numpy(big.astype(np.int64)).to(dev())].cpu().numpy()


def test_bf16_pool_past_4gib(orc, pkv):
    nb = 70_000                                        # 64 KB blocks: 4.59 GB per pool
    x = _inputs(nb, BS * HKV * D * 2, seed=2730)
    print(f"bf16 pool of {nb} blocks, used ids {x['big'].min()}..{x['big'].max()}", flush=True)
    kc, vc = x["k"].copy(), x["v"].copy()
    orc.append(x["kn"], x["vn"], kc, vc, x["compact"], CTX, BS)
    scale = 1.0 / np.sqrt(D)
    ref, _ = orc.paged_attention(x["q"], kc, vc, x["compact"], CTX, scale, block_size=BS,
                                 Hkv=HKV)

    k = _device_pool(x["k"], x["big"], nb, torch.int16)
    v = _device_pool(x["v"], x["big"], nb, torch.int16)
    q, kn, vn = to_dev(x["q"]), to_dev(x["kn"]), to_dev(x["vn"])
    bt, cl = tables_to_dev(x["far"], CTX, BS, nb)

    pkv.paged_kv_append(kn, vn, k, v, bt, cl)
    assert np.array_equal(_blocks(k, x["big"]).view(np.uint16), kc)
    assert np.array_equal(_blocks(v, x["big"]).view(np.uint16), vc)

    out = pkv.paged_decode_attention(q, k, v, bt, cl, scale)
    assert_close(out, ref, "single pass")
    S = 256
    ms = pkv.max_splits_for(int(CTX.max()), S)
    po = torch.empty((B, HQ, ms, D), dtype=torch.float32, device=dev())
    pl = torch.empty((B, HQ, ms), dtype=torch.float32, device=dev())
    pkv.paged_decode_attention(q, k, v, bt, cl, scale, split_tokens=S, partial_out=po,
                               partial_lse=pl)
    assert_close(pkv.split_context_reduce(po, pl, cl, S), ref, "split 256 + reduce")
    ws = pkv.make_workspace(q, k)
    out_b = pkv.paged_decode_attention_balanced(q, k, v, bt, cl, scale, workspace=ws)
    assert_close(out_b, ref, "balanced")

    # whole-block gather of the used blocks
    ids = to_dev(x["big"])
    ko = torch.empty((x["total"], BS, HKV, D), dtype=torch.int16, device=dev())
    vo = torch.empty_like(ko)
    pkv.paged_kv_gather_blocks(k, v, ids, ko, vo)
    assert np.array_equal(ko.cpu().numpy().view(np.uint16), kc)
    assert np.array_equal(vo.cpu().numpy().view(np.uint16), vc)

    # the fused step on the original blocks
    idx = torch.from_numpy(x["big"].astype(np.int64)).to(dev())
    k[idx] = to_dev(x["k"])
    v[idx] = to_dev(x["v"])
    out_f = pkv.paged_append_decode_attention_balanced(q, kn, vn, k, v, bt, cl, scale,
                                                       workspace=ws)
    assert_close(out_f, ref, "fused append + balanced")
    assert np.array_equal(_blocks(k, x["big"]).view(np.uint16), kc)
    assert np.array_equal(_blocks(v, x["big"]).view(np.uint16), vc)
    del k, v, ko, vo
    torch.cuda.empty_cache()


def test_fp8_pool_past_4gib(orc, pkv):
    nb = 140_000                                       # 32 KB blocks: 4.59 GB per pool
    x = _inputs(nb, BS * HKV * D, seed=2731)
    print(f"fp8 pool of {nb} blocks, used ids {x['big'].min()}..{x['big'].max()}", flush=True)
    ks = orc.fp8_block_scales(x["k"], x["compact"], CTX, BS)
    vs = orc.fp8_block_scales(x["v"], x["compact"], CTX, BS)
    kq, vq = orc.fp8_quantize_pool(x["k"], ks), orc.fp8_quantize_pool(x["v"], vs)
    for pool in (kq, vq):                              # poison stays poison as codes
        pool[x["k"] == NAN_BF16] = NAN_E4M3
    kc, vc = kq.copy(), vq.copy()
    orc.append(x["kn"], x["vn"], kc, vc, x["compact"], CTX, BS, kv_dtype="fp8", k_scale=ks,
               v_scale=vs)
    scale = 1.0 / np.sqrt(D)
    ref, _ = orc.paged_attention(x["q"], kc, vc, x["compact"], CTX, scale, block_size=BS,
                                 Hkv=HKV, kv_dtype="fp8", k_scale=ks, v_scale=vs)

    k = _device_pool(kq, x["big"], nb, torch.uint8)
    v = _device_pool(vq, x["big"], nb, torch.uint8)
    idx = torch.from_numpy(x["big"].astype(np.int64)).to(dev())
    ksd = torch.ones((nb, HKV), dtype=torch.float32, device=dev())
    vsd = torch.ones_like(ksd)
    ksd[idx], vsd[idx] = to_dev(ks), to_dev(vs)
    q, kn, vn = to_dev(x["q"]), to_dev(x["kn"]), to_dev(x["vn"])
    bt, cl = tables_to_dev(x["far"], CTX, BS, nb)

    ws = pkv.make_workspace(q, k)
    out = pkv.paged_append_decode_attention_balanced(q, kn, vn, k, v, bt, cl, scale,
                                                     workspace=ws, k_scale=ksd, v_scale=vsd)
    assert np.array_equal(_blocks(k, x["big"]), kc)
    assert np.array_equal(_blocks(v, x["big"]), vc)
    assert_close(out, ref, "fp8 fused append + balanced")
    out_s = pkv.paged_decode_attention(q, k, v, bt, cl, scale, k_scale=ksd, v_scale=vsd)
    assert_close(out_s, ref, "fp8 single pass")
    del k, v
    torch.cuda.empty_cache()
