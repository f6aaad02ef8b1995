"""Pins the oracle's FP8 E4M3FN codec to the format definition and to an
independent implementation (PyTorch's CPU float8_e4m3fn cast).  CPU only.

[B] "Quantized KV Cache" / "FP8 KV cache": E4M3 storage, values divided by a
scale on write and multiplied back on read.
"""
import math

import numpy as np
import pytest
import torch

from synthetic import bf16_bits_from_f32, f32_from_bf16_bits


def test_special_codes(orc):
    assert orc.e4m3_value(0x38) == 1.0
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0xFE) == -448.0
    assert orc.e4m3_value(0x08) == 2.0 ** -6          # smallest normal
    assert orc.e4m3_value(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert orc.e4m3_value(0x01) == 2.0 ** -9          # smallest subnormal
    assert orc.e4m3_value(0x00) == 0.0
    z = orc.e4m3_value(0x80)
    assert z == 0.0 and math.copysign(1.0, z) < 0
    assert math.isnan(orc.e4m3_value(0x7F)) and math.isnan(orc.e4m3_value(0xFF))
    assert orc.e4m3_value(0x40) == 2.0 and orc.e4m3_value(0x30) == 0.5


def test_decode_matches_torch_for_all_codes(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([orc.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def test_positive_codes_strictly_increasing(orc):
    vals = [orc.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def test_encode_inverts_decode(orc):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert orc.e4m3_encode(orc.e4m3_value(c)) == c


def test_midpoints_round_to_even(orc):
    for c in range(0x7E):
        lo, hi = orc.e4m3_value(c), orc.e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # exactly representable in binary32
        want = c if c % 2 == 0 else c + 1
        assert orc.e4m3_encode(float(mid)) == want
        assert orc.e4m3_encode(-float(mid)) == 0x80 | want
        # just off the midpoint goes to the nearer code
        assert orc.e4m3_encode(float(np.nextafter(mid, np.float32(0)))) == c
        assert orc.e4m3_encode(float(np.nextafter(mid, np.float32(1e9)))) == c + 1


def test_saturation_and_nan(orc):
    assert orc.e4m3_encode(1e6) == 0x7E
    assert orc.e4m3_encode(-1e6) == 0xFE
    assert orc.e4m3_encode(449.0) == 0x7E
    assert orc.e4m3_encode(float("inf")) == 0x7E
    assert orc.e4m3_encode(float("-inf")) == 0xFE
    assert orc.e4m3_encode(float("nan")) == 0x7F
    assert orc.e4m3_encode(-0.0) == 0x80
    assert orc.e4m3_encode(2.0 ** -11) == 0x00     # below half the smallest subnormal
    assert orc.e4m3_encode(-(2.0 ** -11)) == 0x80


@pytest.mark.parametrize("scale", [1.0, 0.0078125, 1.0 / 3.0, 7.3, 2.0 ** -12])
def test_quantize_exhaustive_bf16_vs_torch(orc, scale):
    """All 65,536 bf16 inputs: y = x / scale in binary32, then E4M3FN.
    PyTorch rounds to nearest even but turns |y| > 464 into NaN instead of
    saturating, so it is the reference for |y| <= 464 and NaN inputs are
    checked separately."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.e4m3_quantize_array(bits, scale)
    x = torch.from_numpy(f32_from_bf16_bits(bits).copy())
    y = x / torch.tensor(np.float32(scale))
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    yv = y.numpy()
    ok = np.abs(yv) <= 464
    assert np.array_equal(ours[ok], ref[ok])
    big = (np.abs(yv) > 464) & ~np.isnan(yv)
    assert np.all(ours[big & (yv > 0)] == 0x7E) and np.all(ours[big & (yv < 0)] == 0xFE)
    assert np.all(ours[np.isnan(yv)] == 0x7F)


def test_quantize_single_matches_array(orc):
    rng = np.random.default_rng(7)
    bits = bf16_bits_from_f32(rng.standard_normal(2000).astype(np.float32) * 30)
    arr = orc.e4m3_quantize_array(bits, 0.05)
    for i in range(0, 2000, 37):
        assert orc.e4m3_quantize(int(bits[i]), 0.05) == arr[i]


def test_block_scales_reach_full_range(orc):
    """scale = amax / 448 per (block, kv head) over live slots: the largest
    live element of every used (block, head) encodes to +-448."""
    from synthetic import generate, make_workload

    wl = make_workload("fp8_36layers_groups4_b32_ctx2k_8k", B=3, ctx_uniform=(20, 70),
                       max_blocks=8, layers=4)
    inp = generate(wl)
    src = inp.k_pool[0].copy()
    # dead slots (holes, tails) get large finite garbage: it must not set a scale
    dead = np.arange(wl.block_size)[None, :] >= inp.live[:, None]
    src[dead] = bf16_bits_from_f32(np.float32(1000.0))
    sc = orc.fp8_block_scales(src, inp.block_tables, inp.context_lens, wl.block_size)
    codes = orc.fp8_quantize_pool(src, sc)
    mags = np.abs(np.vectorize(orc.e4m3_value)(codes))
    for p in range(inp.num_blocks):
        n = inp.live[p]
        for h in range(wl.Hkv):
            if n == 0:
                assert sc[p, h] == 1.0
                continue
            live_vals = mags[p, :n, h, :]
            finite = live_vals[~np.isnan(live_vals)]
            assert finite.max() == 448.0
            # poisoned live slot (the append position) stays NaN
    assert np.all(codes[np.isnan(f32_from_bf16_bits(src))] == 0x7F)
    assert dead.sum() > 0
