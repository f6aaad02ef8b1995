"""Pins the oracle's block-table validator and the live-slot rule of its
scale builders.  CPU only.

[B] "PagedAttention": a sequence's block table maps its logical blocks to
physical blocks of the pool, and only the last block of a sequence may be
partly filled.  Fixed by that definition, not by the oracle:
  * a table is valid when every sequence fits its row (0 <= T <=
    max_blocks * block_size) and each of its ceil(T / block_size) live
    entries names a block inside the pool [0, num_blocks);
  * entries past the live ones are never read, so any value there is
    valid, and a sequence with T = 0 reads no entry at all;
  * the first offending sequence b is reported as -(1 + b).
The scale and zero-point builders read only the live slots of a block:
finite values planted in the dead tail of a partial block (slots the table
never covers) must not move any scale ([B] "FP8 KV cache", "INT8 KV
cache": the parameters describe the values the block holds).
"""
import numpy as np
import pytest

from synthetic import bf16_bits_from_f32, f32_from_bf16_bits, generate, make_workload

TINY = "tiny_b4_hq8_hkv2_d64_bs16"


def _tables():
    # 3 sequences over a 10-block pool, block size 4, 3 entries per row
    bt = np.array([[7, 2, -1],
                   [0, 9, 5],
                   [3, -1, -1]], dtype=np.int32)
    cl = np.array([6, 12, 1], dtype=np.int32)
    return bt, cl


def test_valid_tables_pass(orc):
    bt, cl = _tables()
    assert orc.check_tables(bt, cl, 4, 10) == 0


def test_unread_entries_may_hold_anything(orc):
    bt, cl = _tables()
    bt[0, 2] = 1 << 30                   # past sequence 0's two live blocks
    bt[2, 1:] = -7
    assert orc.check_tables(bt, cl, 4, 10) == 0
    cl0 = cl.copy()
    cl0[1] = 0                           # an empty sequence reads no entry
    bt[1, :] = -1
    assert orc.check_tables(bt, cl0, 4, 10) == 0


@pytest.mark.parametrize("b,j,value", [(0, 0, -1), (0, 1, 10), (1, 2, -1), (1, 2, 10),
                                       (2, 0, 1 << 20)])
def test_live_entry_outside_the_pool(orc, b, j, value):
    bt, cl = _tables()
    bt[b, j] = value
    assert orc.check_tables(bt, cl, 4, 10) == -(1 + b)


def test_last_partial_block_is_checked(orc):
    # sequence 0 has 6 tokens: its second block is live though only half full
    bt, cl = _tables()
    bt[0, 1] = 10
    assert orc.check_tables(bt, cl, 4, 10) == -1
    # one token more than the live blocks cover makes the next entry live
    bt, cl = _tables()
    cl[0] = 9
    assert orc.check_tables(bt, cl, 4, 10) == -1       # entry 2 is -1
    cl[0] = 8
    assert orc.check_tables(bt, cl, 4, 10) == 0


def test_context_bounds(orc):
    bt, cl = _tables()
    cl[1] = 12                                         # exactly max_blocks * block_size
    assert orc.check_tables(bt, cl, 4, 10) == 0
    cl[1] = 13
    assert orc.check_tables(bt, cl, 4, 10) == -2
    cl[1] = 12
    cl[2] = -1
    assert orc.check_tables(bt, cl, 4, 10) == -3


def test_first_offender_is_reported(orc):
    bt, cl = _tables()
    bt[1, 0] = -1
    bt[2, 0] = -1
    assert orc.check_tables(bt, cl, 4, 10) == -2


def test_generated_workloads_are_valid(orc):
    for name in (TINY, "llama70b_b64_ragged1k_16k_bs32"):
        wl = make_workload(name) if name == TINY else make_workload(name, B=6)
        inp = generate(wl, groups=[])
        assert orc.check_tables(inp.block_tables, inp.context_lens, wl.block_size,
                                inp.num_blocks) == 0


# ------------------------------------------------------- live-slot rule
def _tail_poisoned_pool():
    """The tiny workload's K pool with a large finite value in every dead
    tail slot of every partly filled block, plus the block and kv head
    whose live values are known."""
    inp = generate(make_workload(TINY))
    wl = inp.wl
    src = inp.k_pool[0].copy()
    big = int(bf16_bits_from_f32(np.array([1000.0], np.float32))[0])
    partial = [p for p in range(inp.num_blocks) if 0 < inp.live[p] < wl.block_size]
    assert partial, "the workload must have partly filled blocks"
    for p in partial:
        src[p, inp.live[p]:] = big
    return inp, src, partial


def _live_values(inp, src, p, h):
    v = f32_from_bf16_bits(src[p, :inp.live[p], h]).astype(np.float64)
    return v[np.isfinite(v)]


def test_int8_params_ignore_dead_tail(orc):
    inp, src, partial = _tail_poisoned_pool()
    wl = inp.wl
    for symmetric in (True, False):
        prm = orc.int8_block_params(src, inp.block_tables, inp.context_lens, wl.block_size,
                                    symmetric=symmetric)
        for p in partial:
            for h in range(wl.Hkv):
                v = _live_values(inp, src, p, h)
                sc = prm[p, h, 0]
                if v.size == 0:                 # only the NaN append slot is live
                    assert sc == 1.0, (p, h)
                elif symmetric:
                    assert np.isclose(sc, np.float32(np.abs(v).max()) / np.float32(127),
                                      rtol=1e-6), (p, h)
                elif v.max() > v.min():
                    ref = (np.float32(v.max()) - np.float32(v.min())) / np.float32(255)
                    assert np.isclose(sc, ref, rtol=1e-6), (p, h)


def test_fp8_block_scales_ignore_dead_tail(orc):
    inp, src, partial = _tail_poisoned_pool()
    wl = inp.wl
    sc = orc.fp8_block_scales(src, inp.block_tables, inp.context_lens, wl.block_size)
    for p in partial:
        for h in range(wl.Hkv):
            v = _live_values(inp, src, p, h)
            ref = np.float32(np.abs(v).max()) / np.float32(448) if v.size else 1.0
            assert np.isclose(sc[p, h], ref, rtol=1e-6), (p, h)


@pytest.mark.parametrize("per_tensor", [False, True])
def test_fp8_wide_scales_ignore_dead_tail(orc, per_tensor):
    inp, src, _ = _tail_poisoned_pool()
    wl = inp.wl
    sc = orc.fp8_wide_scales(src, inp.block_tables, inp.context_lens, wl.block_size,
                             per_tensor=per_tensor)
    amax = np.zeros(wl.Hkv)
    for p in range(inp.num_blocks):
        for h in range(wl.Hkv):
            v = _live_values(inp, src, p, h)
            if v.size:
                amax[h] = max(amax[h], np.abs(v).max())
    assert amax.max() < 1000.0
    if per_tensor:
        assert np.isclose(sc[0], np.float32(amax.max()) / np.float32(448), rtol=1e-6)
    else:
        for h in range(wl.Hkv):
            assert np.isclose(sc[h], np.float32(amax[h]) / np.float32(448), rtol=1e-6)
