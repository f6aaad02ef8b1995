"""Structure of the seeded synthetic workloads (CPU only).

[B] "PagedAttention": tables map logical to physical blocks anywhere in
the pool; only a sequence's last block is partial; blocks may be shared.
[A] "What is cross-layer KV sharing": groups of consecutive layers.
"""
import numpy as np
import pytest

from synthetic import WORKLOADS, generate, make_workload
from synthetic.workloads import BF16_QNAN


def _check_structure(inp):
    wl = inp.wl
    bs = wl.block_size
    ctx = inp.context_lens
    assert ctx.dtype == np.int32 and inp.block_tables.dtype == np.int32
    nblk = (ctx + bs - 1) // bs
    refs = {}
    for b in range(wl.B):
        row = inp.block_tables[b]
        assert np.all(row[:nblk[b]] >= 0) and np.all(row[:nblk[b]] < inp.num_blocks)
        assert np.all(row[nblk[b]:] == -1)
        # waste in the last block is at most block_size - 1
        assert 0 <= nblk[b] * bs - ctx[b] <= bs - 1
        for j in range(nblk[b]):
            refs.setdefault(int(row[j]), set()).add((b, j))
    return refs


@pytest.mark.parametrize("name", ["tiny_b4_hq8_hkv2_d64_bs16"])
def test_tiny_layout(name):
    inp = generate(WORKLOADS[name])
    refs = _check_structure(inp)
    assert list(inp.context_lens) == [1, 17, 100, 513]
    assert inp.num_blocks == 64 and len(refs) == 43
    holes = [p for p in range(64) if p not in refs]
    assert len(holes) == 21
    for p in holes:
        assert np.all(inp.k_pool[0][p] == BF16_QNAN) and np.all(inp.v_pool[0][p] == BF16_QNAN)


def test_ragged_pool_has_ten_percent_holes():
    wl = make_workload("llama70b_b64_ragged1k_16k_bs32", B=64)
    # only the tables are needed; draw them without the big pools
    inp = generate(wl, groups=[])
    refs = _check_structure(inp)
    holes = inp.num_blocks - len(refs)
    assert abs(holes / inp.num_blocks - 0.10) < 0.002
    assert inp.context_lens.min() >= 1024 and inp.context_lens.max() <= 16384
    # holes are scattered, not a tail of the pool
    hole_ids = sorted(set(range(inp.num_blocks)) - set(refs))
    assert hole_ids[0] < inp.num_blocks // 4 and hole_ids[-1] > 3 * inp.num_blocks // 4


def test_shared_prefix_tables():
    wl = WORKLOADS["llama70b_b4_ctx32k_split512_prefix2k"]
    inp = generate(wl, groups=[])
    refs = _check_structure(inp)
    assert inp.num_blocks == 7808 == len(refs)
    for j in range(128):
        assert len(set(inp.block_tables[:, j])) == 1
    assert len(set(inp.block_tables[:, 128])) == 4


def test_exact_pool_and_groups():
    wl = WORKLOADS["fp8_36layers_groups4_b32_ctx2k_8k"]
    inp = generate(wl, groups=[])
    refs = _check_structure(inp)
    assert inp.num_blocks == len(refs)
    assert wl.groups == 9 and wl.layers_per_group == 4
    assert inp.query.shape == (36, 32, 32, 128)


def test_deterministic_and_seed_sensitive():
    wl = make_workload("tiny_b4_hq8_hkv2_d64_bs16")
    a, b = generate(wl), generate(wl)
    assert np.array_equal(a.k_pool[0], b.k_pool[0]) and np.array_equal(a.block_tables,
                                                                      b.block_tables)
    c = generate(wl, seed=wl.seed + 1000)
    assert not np.array_equal(a.k_pool[0], c.k_pool[0])


def test_poison_positions():
    inp = generate(WORKLOADS["tiny_b4_hq8_hkv2_d64_bs16"])
    wl = inp.wl
    for b in range(wl.B):
        T = int(inp.context_lens[b])
        p = inp.block_tables[b, (T - 1) // wl.block_size]
        assert np.all(inp.k_pool[0][p, (T - 1) % wl.block_size] == BF16_QNAN)
        if T >= 2:
            p2 = inp.block_tables[b, (T - 2) // wl.block_size]
            assert not np.any(inp.k_pool[0][p2, (T - 2) % wl.block_size] == BF16_QNAN)


def test_value_distribution():
    from synthetic import f32_from_bf16_bits

    inp = generate(make_workload("llama8b_b32_ctx4096_bs16", B=2, ctx_fixed=(4096, 4096)))
    k = f32_from_bf16_bits(inp.k_pool[0]).astype(np.float64)
    k = k[np.isfinite(k)]
    assert abs(k.mean()) < 0.01 and abs(k.std() - 1.0) < 0.01
    q = f32_from_bf16_bits(inp.query).astype(np.float64)
    assert abs(q.std() * np.sqrt(128) - 1.0) < 0.05


def test_multiquery_layout_and_poison():
    from synthetic import generate_multiquery

    wl = WORKLOADS["tiny_mq_b4_hq8_hkv2_d64_bs16"]
    mq = generate_multiquery(wl)
    ctx = mq.base.context_lens
    assert (mq.query_lens >= 0).all() and (mq.query_lens <= ctx).all()
    assert mq.query_lens[0] == 1                      # clipped to T_0 = 1
    assert mq.query_start[0] == 0 and np.array_equal(np.diff(mq.query_start), mq.query_lens)
    assert mq.k_rows[0].shape == (mq.rows, wl.Hkv, wl.D)
    assert mq.query.shape == (1, mq.rows, wl.Hq, wl.D)
    for b in range(wl.B):
        T, q = int(ctx[b]), int(mq.query_lens[b])
        for t in range(T):
            p = mq.base.block_tables[b, t // wl.block_size]
            row = mq.base.k_pool[0][p, t % wl.block_size]
            assert (row == 0x7FC0).all() == (t >= T - q), (b, t)
    again = generate_multiquery(wl)
    assert np.array_equal(again.query, mq.query) and np.array_equal(again.k_rows[0], mq.k_rows[0])
    fixed = generate_multiquery(wl, query_lens=np.array([5, 5, 5, 5]))
    assert list(fixed.query_lens) == [1, 5, 5, 5]
