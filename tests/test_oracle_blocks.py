"""Pins the oracle's whole-block moves (gather / scatter / copy).  CPU only.

Fixed by plain definitions: a gathered block equals NumPy's own indexing
of the pool, scatter is its inverse, a copied block equals its source and
nothing else moves.  ([C] "When the cache fills": swapping a preempted
sequence's blocks to host memory and back; [B] "PagedAttention" block
sharing, whose copy-on-write copies a block.)
"""
import numpy as np
import pytest

from synthetic import generate, make_workload

TINY = "tiny_b4_hq8_hkv2_d64_bs16"


@pytest.fixture(scope="module")
def pool():
    inp = generate(make_workload(TINY))
    return inp.k_pool[0]


def test_gather_is_indexing(orc, pool):
    ids = np.array([5, 0, 63, 5, 17], dtype=np.int32)
    out = orc.gather_blocks(pool, ids)
    assert out.view(np.uint16).tobytes() == pool[ids].tobytes()


def test_scatter_inverts_gather(orc, pool):
    rng = np.random.default_rng(3)
    ids = rng.permutation(pool.shape[0])[:20].astype(np.int32)
    blocks = orc.gather_blocks(pool, ids)
    dst = np.zeros_like(pool)
    orc.scatter_blocks(blocks, ids, dst)
    mask = np.zeros(pool.shape[0], dtype=bool)
    mask[ids] = True
    assert dst[mask].tobytes() == pool[mask].tobytes()
    assert not dst[~mask].any()


def test_copy_moves_exactly_the_listed_blocks(orc, pool):
    p = pool.copy()
    src = np.array([1, 2, 3], dtype=np.int32)
    dst = np.array([10, 40, 0], dtype=np.int32)
    orc.copy_blocks(p, src, dst)
    for s, d in zip(src, dst):
        assert p[d].tobytes() == pool[s].tobytes()
    keep = np.setdiff1d(np.arange(pool.shape[0]), dst)
    assert p[keep].tobytes() == pool[keep].tobytes()


def test_scale_rows_are_blocks_too(orc):
    sc = np.arange(64 * 2, dtype=np.float32).reshape(64, 2)
    ids = np.array([7, 3], dtype=np.int32)
    assert np.array_equal(orc.gather_blocks(sc, ids), sc[ids])
