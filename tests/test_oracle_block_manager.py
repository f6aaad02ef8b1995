"""Pins the reference block manager (oracle/block_manager.py).  CPU only.

Each check is fixed by the pages or follows from what a block table must
do, not by the model itself:
  * [B] "Prefix Caching" worked example: three requests with one 500-token
    system prompt compute 500 prompt tokens in total instead of 1500;
  * [B] "PagedAttention": only the last block of a sequence is partly
    filled (ceil(T / bs) blocks); a retiring request returns every block;
  * [A] "How does prefix caching work": the key is cumulative -- equal block
    content after a different prefix is not a hit; matching stops at the
    first miss;
  * [C] "When the cache fills": unused cached blocks are evicted least
    recently used first, and only when no block is free;
  * content: a simulated pool written through the tables (token ids as the
    cached values, copy-on-write copies applied) reads back every
    sequence's tokens exactly, through forks, shared prefixes and evictions;
  * an operation that cannot get its blocks changes nothing.
"""
import copy
import importlib.util
import os
import random

import pytest

if os.environ.get("PKV_ORACLE_BM"):          # a planted-mistake copy (mutant test)
    _spec = importlib.util.spec_from_file_location("bm_mutant", os.environ["PKV_ORACLE_BM"])
    _mod = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(_mod)
    NoSpace, RefBlockManager = _mod.NoSpace, _mod.RefBlockManager
else:
    from oracle.block_manager import NoSpace, RefBlockManager


class Pool:
    """Host stand-in for the device cache: pool[block][slot] = token id."""

    def __init__(self, m: RefBlockManager):
        self.m = m
        self.data = [[None] * m.bs for _ in range(m.num_blocks)]

    def _write(self, seq, start):
        m = self.m
        for copy_ in m.take_copies():
            src, dst, n = copy_
            self.data[dst][:n] = self.data[src][:n]
        toks, table = m.tokens[seq], m.tables[seq]
        for t in range(start, len(toks)):
            self.data[table[t // m.bs]][t % m.bs] = toks[t]

    def add(self, seq, toks):
        cached = self.m.add(seq, toks)
        self._write(seq, cached)
        return cached

    def append(self, seq, toks):
        n = len(self.m.tokens[seq])
        self.m.append(seq, toks)
        self._write(seq, n)

    def check(self):
        m = self.m
        for seq, toks in m.tokens.items():
            table = m.tables[seq]
            assert len(table) == (len(toks) + m.bs - 1) // m.bs
            got = [self.data[table[t // m.bs]][t % m.bs] for t in range(len(toks))]
            assert got == toks, seq


def _refs_consistent(m: RefBlockManager):
    count = [0] * m.num_blocks
    for table in m.tables.values():
        for b in table:
            count[b] += 1
    assert count == m.ref
    assert sorted(m.free + m.lru + [b for b in range(m.num_blocks) if m.ref[b] > 0]) == \
        list(range(m.num_blocks))
    for k, b in m.cache.items():
        assert m.key[b] == k


@pytest.mark.parametrize("bs,expected", [(20, [500, 0, 0]), (4, [500, 0, 0]),
                                         (16, [500, 4, 4])])
def test_worked_example_three_requests(bs, expected):
    """[B] "Prefix Caching": 3 requests sharing a 500-token system prompt.
    With block-granular caching of full blocks ([B] "How vLLM implements
    automatic prefix caching"), a block size that does not divide 500 leaves
    the 4-token tail of the prompt to be recomputed by every request."""
    m = RefBlockManager(1000, bs)
    pool = Pool(m)
    system = list(range(1000, 1500))
    computed_prompt = []
    for r in range(3):
        user = [5000 + 100 * r + i for i in range(37)]
        cached = pool.add(r, system + user)
        computed_prompt.append(max(0, 500 - cached))
        assert cached <= 500
    assert computed_prompt == expected
    if bs in (20, 4):
        assert sum(computed_prompt) == 500 and 3 * 500 - sum(computed_prompt) == 1000
    pool.check()
    _refs_consistent(m)


def test_only_the_last_block_is_partial_and_release_returns_all():
    rng = random.Random(1)
    m = RefBlockManager(400, 16)
    pool = Pool(m)
    for s in range(20):
        pool.add(s, [rng.randrange(50000) for _ in range(rng.randrange(1, 200))])
    pool.check()
    used = sum(len(t) for t in m.tables.values())
    assert used == sum((len(t) + 15) // 16 for t in m.tokens.values())
    for s in range(20):
        m.release(s)
    assert all(r == 0 for r in m.ref)
    assert m.num_free() + m.num_evictable() == 400
    _refs_consistent(m)


def test_key_is_cumulative():
    m = RefBlockManager(64, 4)
    A, Bb, C = [1, 2, 3, 4], [5, 6, 7, 8], [9, 9, 9, 9]
    assert m.add(0, A + Bb + [10]) == 0
    # same second block after a different first block: no hit at all
    assert m.add(1, C + Bb + [10]) == 0
    assert m.tables[1][1] != m.tables[0][1]
    # same prefix: both blocks hit
    assert m.add(2, A + Bb + [11, 12]) == 8
    assert m.tables[2][:2] == m.tables[0][:2]
    # first block hits, second misses: matching stops there
    assert m.add(3, A + C + Bb + [1]) == 4
    assert m.tables[3][0] == m.tables[0][0] and m.tables[3][2] != m.tables[0][1]
    _refs_consistent(m)


def test_last_token_is_always_computed():
    m = RefBlockManager(16, 4)
    m.add(0, list(range(8)))
    assert m.add(1, list(range(8))) == 4          # block 1 holds the last token
    assert m.add(2, list(range(9))) == 8
    _refs_consistent(m)


def test_lru_eviction_only_when_nothing_is_free():
    m = RefBlockManager(6, 2)
    m.add(0, [1, 2, 3, 4, 9])       # blocks 0, 1 keyed; 2 partial
    m.add(1, [5, 6, 7])             # block 3 keyed; 4 partial
    m.release(0)                    # released last block first: 2 -> free, 1, 0 -> lru
    m.release(1)                    # 4 -> free, 3 -> lru
    assert m.lru == [1, 0, 3] and sorted(m.free) == [2, 4, 5]
    # a re-hit takes a block off the LRU list
    assert m.add(2, [1, 2, 8]) == 2
    assert m.tables[2][0] == 0 and m.lru == [1, 3]
    # the two free blocks (4, 5) are used before anything is evicted
    m.add(3, [20, 21, 22, 23])
    assert m.tables[3] == [4, 5] and m.lru == [1, 3] and m.num_free() == 0
    # the next allocation evicts the least recently released block (1)
    m.append(3, [26])
    assert m.tables[3][-1] == 1 and m.lru == [3]
    assert (0, (1, 2, 3, 4)) not in m.cache        # its key is gone
    with pytest.raises(NoSpace):                   # 2 new blocks, 1 evictable
        m.add(4, [1, 2, 3, 4, 0])
    assert m.add(4, [1, 2, 3]) == 2                # block 0 hits, block 3 evicted
    assert m.tables[4] == [0, 3] and m.lru == []
    _refs_consistent(m)


def test_fork_copy_on_write_keeps_every_sequence_intact():
    m = RefBlockManager(64, 4)
    pool = Pool(m)
    pool.add(0, [1, 2, 3, 4, 5, 6])
    m.fork(0, 1)
    m.fork(0, 2)
    pool.append(1, [70])            # shared partial block: copied first
    pool.append(2, [80, 81])
    pool.append(0, [90, 91, 92])
    pool.check()
    assert m.tables[0][0] == m.tables[1][0] == m.tables[2][0]
    assert len({m.tables[s][1] for s in range(3)}) == 3
    _refs_consistent(m)


def test_no_space_changes_nothing():
    m = RefBlockManager(5, 4)
    m.add(0, list(range(12)))
    before = copy.deepcopy(m.__dict__)
    with pytest.raises(NoSpace):
        m.add(1, list(range(100, 121)))   # needs 6 blocks
    assert m.__dict__ == before
    m.add(1, list(range(100, 105)))       # 2 blocks: fits
    before = copy.deepcopy(m.__dict__)
    with pytest.raises(NoSpace):
        m.append(1, list(range(10)))
    assert m.__dict__ == before


def test_random_traffic_content_and_counts():
    """Seeded random mix of add / append / fork / release over prompts that
    share prefixes, in a pool small enough to force eviction."""
    rng = random.Random(7)
    m = RefBlockManager(120, 8)
    pool = Pool(m)
    prefixes = [[rng.randrange(1000) for _ in range(rng.randrange(8, 60))] for _ in range(4)]
    live, nxt = [], 0
    for _ in range(400):
        op = rng.random()
        try:
            if op < 0.35 or not live:
                toks = rng.choice(prefixes)[:rng.randrange(1, 60)] + \
                    [rng.randrange(1000) for _ in range(rng.randrange(0, 20))]
                if not toks:
                    continue
                pool.add(nxt, toks)
                live.append(nxt)
                nxt += 1
            elif op < 0.7:
                pool.append(rng.choice(live), [rng.randrange(1000) for _ in range(rng.randrange(1, 12))])
            elif op < 0.8:
                m.fork(rng.choice(live), nxt)
                live.append(nxt)
                nxt += 1
            else:
                s = live.pop(rng.randrange(len(live)))
                m.release(s)
        except NoSpace:
            pass
        pool.check()
        _refs_consistent(m)
    assert m.cache, "no prefix block was ever cached"
