"""Pins the oracle's INT8 and per-head / per-tensor FP8 cache formats.
CPU only.

[B] "INT8 KV cache": symmetric or asymmetric integer quantisation with a
scale and a zero point; [B] "FP8 KV cache": a per-tensor or per-head scale.
Fixed by the definitions, not by the oracle:
  * int8 codes of exact multiples scale * (k - zp) are k; halves round to
    the even integer; out-of-range values clamp to 0 / 255; NaN -> 0;
  * dequantisation error of an in-range value is at most scale / 2 (plus
    the binary32 division's rounding);
  * symmetric parameters put 0 at code 128 and +-amax at 128 +- 127;
    asymmetric parameters put min near code 0 and max near code 255;
  * per-head / per-tensor fp8 scales are the amax over the live tokens of
    that head / of everything, / 448; the amax element encodes to +-448;
  * attention over every format equals dense NumPy attention on values
    dequantised here (int8: scale * (u - zp); fp8: PyTorch's E4M3 decode).
"""
import math

import numpy as np
import pytest

from synthetic import bf16_bits_from_f32, f32_from_bf16_bits, generate, make_workload

TINY = "tiny_b4_hq8_hkv2_d64_bs16"


def _bf(x):
    return int(bf16_bits_from_f32(np.array([x], dtype=np.float32))[0])


@pytest.mark.parametrize("scale,zp", [(0.5, 128.0), (0.03125, 7.0), (2.0, 255.0), (1.0, 0.0)])
def test_int8_exact_multiples(orc, scale, zp):
    for k in range(0, 256, 5):
        x = scale * (k - zp)
        if _bf(x) != bf16_bits_from_f32(np.array([x], np.float32))[0] or \
                float(f32_from_bf16_bits(np.array([_bf(x)]))[0]) != x:
            continue                    # not exact in bf16: skip
        assert orc.int8_quantize(_bf(x), scale, zp) == k


def test_int8_ties_clamp_nan(orc):
    assert orc.int8_quantize(_bf(2.5), 1.0, 0.0) == 2        # tie -> even
    assert orc.int8_quantize(_bf(3.5), 1.0, 0.0) == 4
    assert orc.int8_quantize(_bf(-2.5), 1.0, 128.0) == 126   # -2 + 128
    assert orc.int8_quantize(_bf(1000.0), 1.0, 128.0) == 255
    assert orc.int8_quantize(_bf(-1000.0), 1.0, 128.0) == 0
    assert orc.int8_quantize(0x7FC0, 1.0, 128.0) == 0        # NaN
    assert orc.int8_quantize(_bf(0.0), 0.25, 128.0) == 128


def test_int8_error_bound(orc):
    rng = np.random.default_rng(1)
    for scale, zp in [(0.02, 128.0), (0.013, 40.0)]:
        lo, hi = scale * (0 - zp), scale * (255 - zp)
        xs = bf16_bits_from_f32(rng.uniform(lo, hi, 2000).astype(np.float32))
        for b in xs:
            x = float(f32_from_bf16_bits(np.array([b]))[0])
            u = orc.int8_quantize(int(b), scale, zp)
            assert abs(scale * (u - zp) - x) <= scale * 0.5 * (1 + 1e-6), (x, u)


@pytest.mark.parametrize("symmetric", [True, False])
def test_int8_block_params(orc, symmetric):
    inp = generate(make_workload(TINY))
    wl = inp.wl
    src = inp.k_pool[0]
    prm = orc.int8_block_params(src, inp.block_tables, inp.context_lens, wl.block_size,
                                symmetric=symmetric)
    p, h = int(inp.block_tables[3, 0]), 1           # a full block of the longest sequence
    vals = f32_from_bf16_bits(src[p, :, h]).astype(np.float64)
    sc, zp = prm[p, h]
    if symmetric:
        assert zp == 128.0 and np.isclose(sc, np.abs(vals).max() / 127, rtol=1e-6)
        i = np.unravel_index(np.argmax(np.abs(vals)), vals.shape)
        u = orc.int8_quantize(int(src[p, i[0], h, i[1]]), sc, zp)
        assert u in (1, 255)
    else:
        assert np.isclose(sc, (vals.max() - vals.min()) / 255, rtol=1e-6)
        i_lo = np.unravel_index(np.argmin(vals), vals.shape)
        i_hi = np.unravel_index(np.argmax(vals), vals.shape)
        assert orc.int8_quantize(int(src[p, i_lo[0], h, i_lo[1]]), sc, zp) <= 1
        assert orc.int8_quantize(int(src[p, i_hi[0], h, i_hi[1]]), sc, zp) >= 254


@pytest.mark.parametrize("per_tensor", [False, True])
def test_fp8_wide_scales(orc, per_tensor):
    inp = generate(make_workload(TINY))
    wl = inp.wl
    src = inp.k_pool[0]
    sc = orc.fp8_wide_scales(src, inp.block_tables, inp.context_lens, wl.block_size,
                             per_tensor=per_tensor)
    live = np.arange(wl.block_size)[None, :] < inp.live[:, None]        # [nb, bs]
    vals = f32_from_bf16_bits(src).astype(np.float64)
    vals = np.where(live[:, :, None, None], np.abs(vals), 0.0)
    vals = np.nan_to_num(vals, nan=0.0)
    if per_tensor:
        assert sc.shape == (1,) and np.isclose(sc[0], vals.max() / 448, rtol=1e-6)
    else:
        assert sc.shape == (wl.Hkv,)
        for h in range(wl.Hkv):
            assert np.isclose(sc[h], vals[:, :, h].max() / 448, rtol=1e-6)
    # the amax element (of head 0, or of everything) encodes to +-448
    kind = "fp8_tensor" if per_tensor else "fp8_head"
    codes = orc.quantize_pool(src, sc, kind)
    if per_tensor:
        i = np.unravel_index(np.argmax(vals), vals.shape)
        assert codes[i] & 0x7F == 0x7E
    else:
        i = np.unravel_index(np.argmax(vals[:, :, 0]), vals[:, :, 0].shape)
        assert codes[i[0], i[1], 0, i[2]] & 0x7F == 0x7E


def _dequant(orc, codes, sc, kind):
    import torch

    if kind == "int8":
        return sc[..., 0][:, None, :, None] * (codes.astype(np.float64)
                                               - sc[..., 1][:, None, :, None])
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if kind == "fp8_head":
        return v * sc.astype(np.float64)[None, None, :, None]
    return v * float(sc[0])


@pytest.mark.parametrize("kind", ["int8", "int8_sym", "fp8_head", "fp8_tensor"])
def test_attention_matches_dense_on_dequantised_values(orc, kind):
    wl = make_workload("fp8_36layers_groups4_b32_ctx2k_8k", B=3, ctx_uniform=(20, 90),
                       max_blocks=8, layers=4, Hq=8, Hkv=2, D=64)
    inp = generate(wl)
    dtype = "int8" if kind.startswith("int8") else kind
    sk = []
    for src in (inp.k_pool[0], inp.v_pool[0]):
        if dtype == "int8":
            sk.append(orc.int8_block_params(src, inp.block_tables, inp.context_lens,
                                            wl.block_size, symmetric=(kind == "int8_sym")))
        else:
            sk.append(orc.fp8_wide_scales(src, inp.block_tables, inp.context_lens,
                                          wl.block_size, per_tensor=(kind == "fp8_tensor")))
    kc = orc.quantize_pool(inp.k_pool[0], sk[0], dtype)
    vc = orc.quantize_pool(inp.v_pool[0], sk[1], dtype)
    orc.append(inp.k_new[0], inp.v_new[0], kc, vc, inp.block_tables, inp.context_lens,
               wl.block_size, kv_dtype=dtype, k_scale=sk[0], v_scale=sk[1])
    out, lse = orc.paged_attention(inp.query[0], kc, vc, inp.block_tables, inp.context_lens,
                                   inp.scale, block_size=wl.block_size, Hkv=wl.Hkv,
                                   kv_dtype=dtype, k_scale=sk[0], v_scale=sk[1])
    kd, vd = _dequant(orc, kc, sk[0], dtype), _dequant(orc, vc, sk[1], dtype)
    q = f32_from_bf16_bits(inp.query[0]).astype(np.float64)
    for b in range(wl.B):
        T = int(inp.context_lens[b])
        t = np.arange(T)
        phys = inp.block_tables[b][t // wl.block_size]
        K, V = kd[phys, t % wl.block_size], vd[phys, t % wl.block_size]
        for hq in range(wl.Hq):
            s = float(inp.scale) * (K[:, hq // wl.G] @ q[b, hq])
            w = np.exp(s - s.max())
            ref = (w[:, None] * V[:, hq // wl.G]).sum(0) / w.sum()
            np.testing.assert_allclose(out[b, hq], ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, hq], s.max() + math.log(w.sum()), atol=1e-12)
