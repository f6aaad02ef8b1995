"""GPU parity of paged_kv_append: bit-exact against the oracle's scatter.

[B] "What the KV Cache Stores and Why" (the new token's K, V are written
once); [B] "PagedAttention" (slot addressing); [B] "FP8 KV cache"
(quantise on write).  Every byte the append must not touch is compared
too (the whole pool is checked).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DeviceInputs, bits16, fp8_group, host_appended, tables_to_dev, to_dev
from synthetic import generate, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_273_amd as m

    return m


@pytest.mark.parametrize("name,over", [
    ("tiny_b4_hq8_hkv2_d64_bs16", {}),
    ("llama8b_b32_ctx4096_bs16", {"ctx_fixed": tuple(range(1, 33)), "max_blocks": 4}),
    ("llama70b_b64_ragged1k_16k_bs32", {"ctx_uniform": (1, 700), "max_blocks": 22}),
])
def test_bf16_append_bit_exact(orc, pkv, name, over):
    inp = generate(make_workload(name, **over))
    print(f"append bf16 {name} {over}", flush=True)
    d = DeviceInputs(inp)
    pkv.paged_kv_append(d.k_new, d.v_new, d.k, d.v, d.bt, d.cl)
    torch.cuda.synchronize()
    kp, vp = host_appended(orc, inp)
    assert np.array_equal(bits16(d.k), kp)
    assert np.array_equal(bits16(d.v), vp)


def test_bf16_append_full_shape(orc, pkv):
    """Llama-3.1-8B shape: 32 sequences x 4096 tokens, 8192-block pool."""
    inp = generate(make_workload("llama8b_b32_ctx4096_bs16"))
    d = DeviceInputs(inp)
    pkv.paged_kv_append(d.k_new, d.v_new, d.k, d.v, d.bt, d.cl)
    torch.cuda.synchronize()
    kp, vp = host_appended(orc, inp)
    assert np.array_equal(bits16(d.k), kp) and np.array_equal(bits16(d.v), vp)


def test_zero_length_sequences_are_skipped(orc, pkv):
    inp = generate(make_workload("tiny_b4_hq8_hkv2_d64_bs16"))
    cl = inp.context_lens.copy()
    cl[1] = 0
    cl[3] = 0
    inp.context_lens = cl
    d = DeviceInputs(inp)
    pkv.paged_kv_append(d.k_new, d.v_new, d.k, d.v, d.bt, d.cl)
    torch.cuda.synchronize()
    kp, vp = host_appended(orc, inp)
    assert np.array_equal(bits16(d.k), kp) and np.array_equal(bits16(d.v), vp)


def test_fp8_append_bit_exact(orc, pkv):
    wl = make_workload("fp8_36layers_groups4_b32_ctx2k_8k", ctx_uniform=(1, 200), max_blocks=13,
                       layers=4)
    inp = generate(wl)
    kc, vc, ks, vs = fp8_group(orc, inp)
    d = DeviceInputs(inp, k_pool=kc, v_pool=vc, k_scale=ks, v_scale=vs)
    pkv.paged_kv_append(d.k_new, d.v_new, d.k, d.v, d.bt, d.cl, k_scale=d.ks, v_scale=d.vs)
    torch.cuda.synchronize()
    kp, vp = host_appended(orc, inp, kv_dtype="fp8", k_pool=kc, v_pool=vc, ks=ks, vs=vs)
    assert np.array_equal(d.k.cpu().numpy(), kp) and np.array_equal(d.v.cpu().numpy(), vp)


@pytest.mark.parametrize("scales", [(1.0, 0.0078125, 1.0 / 3.0, 7.3, 2.0 ** -12, 1e-30,
                                     3e4, 0.37)])
def test_fp8_encode_exhaustive(orc, pkv, scales):
    """All 65,536 bf16 bit patterns (NaN, inf, subnormals included) through
    the fp8 append, under several block scales: codes equal the oracle's."""
    B, Hkv, D, bs = 64, 8, 128, 16
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(B, Hkv, D)
    for sc in scales:
        print(f"fp8 exhaustive scale={sc}", flush=True)
        nb = B
        tables = np.arange(B, dtype=np.int32).reshape(B, 1)
        ctx = np.full(B, 1, dtype=np.int32)
        ks = np.full((nb, Hkv), sc, dtype=np.float32)
        ks[::3] = np.float32(sc * 3.0)
        vs = np.full((nb, Hkv), np.float32(1.0) / np.float32(sc), dtype=np.float32)
        kc = np.zeros((nb, bs, Hkv, D), dtype=np.uint8)
        vc = np.zeros((nb, bs, Hkv, D), dtype=np.uint8)
        vbits = bits[::-1].copy()
        dk, dv = to_dev(kc), to_dev(vc)
        dbt, dcl = tables_to_dev(tables, ctx, bs, nb)
        pkv.paged_kv_append(to_dev(bits), to_dev(vbits), dk, dv, dbt, dcl,
                            k_scale=to_dev(ks), v_scale=to_dev(vs))
        torch.cuda.synchronize()
        orc.append(bits, vbits, kc, vc, tables, ctx, bs, kv_dtype="fp8", k_scale=ks,
                   v_scale=vs)
        gk, gv = dk.cpu().numpy(), dv.cpu().numpy()
        if not np.array_equal(gk, kc):
            i = np.argwhere(gk != kc)[0]
            raise AssertionError(f"scale {sc}: K code mismatch at {tuple(i)}: gpu {gk[tuple(i)]:#x}"
                                 f" oracle {kc[tuple(i)]:#x}")
        assert np.array_equal(gv, vc)


def test_append_rejects_bad_arguments(pkv):
    inp = generate(make_workload("tiny_b4_hq8_hkv2_d64_bs16"))
    d = DeviceInputs(inp)
    L = pkv.lib()
    st = L.paged_kv_append(d.k_new.data_ptr(), d.v_new.data_ptr(), d.k.data_ptr(),
                           d.v.data_ptr(), None, None, d.bt.data_ptr(), 33, d.cl.data_ptr(),
                           4, 2, 48, 16, 64, 0, None)
    assert st == pkv.PKV_EUNSUPPORTED
    st = L.paged_kv_append(d.k_new.data_ptr(), d.v_new.data_ptr(), d.k.data_ptr(),
                           d.v.data_ptr(), None, None, d.bt.data_ptr(), 33, d.cl.data_ptr(),
                           4, 2, 64, 16, 64, 1, None)
    assert st == pkv.PKV_EINVAL      # fp8 without scales
