"""Reference model of the paged block manager and prefix cache --
TEST INFRASTRUCTURE ONLY (tests/ may import it; the product never does).

Plain Python, written for a reader to check against the pages by eye:

  * [B] "PagedAttention": a pool of equal-size physical blocks; a
    per-sequence table maps logical block j to a physical block; only the
    last block of a sequence is partly filled; any free block serves any
    request; a retiring request returns its blocks to the free pool;
    identical content may share physical blocks.
  * [A] "How does prefix caching work" and [B] "How vLLM implements
    automatic prefix caching": every FULL block is keyed by the content of
    the whole prefix up to its end (a cumulative key); a new request walks
    its prefix block by block and maps each matching block into its table;
    the first block that does not match, and everything after it, is
    computed.
  * [C] "When the cache fills": cached prefix blocks that no sequence uses
    are evicted least-recently-used first.
  * [A] "What is cross-layer KV sharing": the cumulative key is taken per
    layer group, not per layer: one table (hence one key per block) serves
    every group of a model, and `namespace` keeps caches whose contents
    differ for the same tokens apart.

Here the key is the exact tuple (namespace, tokens[0 : end of block]) -- no
hash function at all -- so the model is exact by construction.

Policy choices the pages leave open (the library implements the same):
  * a new block is the lowest-numbered free block; only when no block is
    free is the least recently released cached block evicted (its key is
    dropped);
  * a sequence's blocks are released last logical block first, so a
    sequence's deeper blocks are evicted before its shallower ones;
  * a prompt of n tokens reuses at most the full blocks inside its first
    n - 1 tokens (the last token is always computed);
  * a block is keyed when it becomes full; if its key is already held by
    another block, the new block stays unkeyed (private);
  * appending to a partly filled block that other sequences share (after
    fork) first copies it to a new block (copy-on-write); the copy is
    reported as (source, destination, valid tokens);
  * an operation that needs more blocks than are free or evictable fails
    and changes nothing.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple


class NoSpace(Exception):
    pass


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int, namespace: int = 0):
        self.num_blocks = num_blocks
        self.bs = block_size
        self.ns = namespace
        self.ref = [0] * num_blocks
        self.key: List[Optional[tuple]] = [None] * num_blocks   # key a block is cached under
        self.free = list(range(num_blocks))                      # kept sorted
        self.lru: List[int] = []                                 # released cached blocks, oldest first
        self.cache: Dict[tuple, int] = {}
        self.tables: Dict[int, List[int]] = {}
        self.tokens: Dict[int, List[int]] = {}
        self.copies: List[Tuple[int, int, int]] = []

    # ------------------------------------------------------------ helpers
    def _key(self, toks, end):
        return (self.ns, tuple(toks[:end]))

    def _available(self):
        return len(self.free) + len(self.lru)

    def _allocate(self) -> int:
        if self.free:
            self.free.sort()
            return self.free.pop(0)
        victim = self.lru.pop(0)
        del self.cache[self.key[victim]]
        self.key[victim] = None
        return victim

    def _take(self, blk):
        if self.ref[blk] == 0:
            self.lru.remove(blk)
        self.ref[blk] += 1

    def _register(self, blk, toks, end):
        k = self._key(toks, end)
        if k not in self.cache:
            self.cache[k] = blk
            self.key[blk] = k

    def _release(self, blk):
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            if self.key[blk] is not None:
                self.lru.append(blk)
            else:
                self.free.append(blk)

    # ------------------------------------------------------------ operations
    def add(self, seq: int, toks: List[int]) -> int:
        """New sequence with prompt toks; returns the number of leading
        tokens whose KV is already cached (a multiple of the block size)."""
        assert seq not in self.tables and len(toks) >= 1
        bs = self.bs
        matched = []
        for j in range((len(toks) - 1) // bs):
            blk = self.cache.get(self._key(toks, (j + 1) * bs))
            if blk is None:
                break
            matched.append(blk)
        nblk = (len(toks) + bs - 1) // bs
        in_lru = sum(1 for b in matched if self.ref[b] == 0)
        if nblk - len(matched) > self._available() - in_lru:
            raise NoSpace()
        for b in matched:
            self._take(b)
        table = list(matched)
        for j in range(len(matched), nblk):
            blk = self._allocate()
            self.ref[blk] = 1
            table.append(blk)
            if (j + 1) * bs <= len(toks):
                self._register(blk, toks, (j + 1) * bs)
        self.tables[seq] = table
        self.tokens[seq] = list(toks)
        return len(matched) * bs

    def append(self, seq: int, toks: List[int]) -> None:
        """Extends a sequence by the given tokens (decode steps, or a chunk)."""
        table, have = self.tables[seq], self.tokens[seq]
        bs = self.bs
        n = len(have)
        need = 0
        if n % bs != 0 and toks and self.ref[table[-1]] > 1:
            need += 1                                   # copy-on-write
        need += (n + len(toks) + bs - 1) // bs - (n + bs - 1) // bs
        if need > self._available():
            raise NoSpace()
        for t in toks:
            if n % bs == 0:
                blk = self._allocate()
                self.ref[blk] = 1
                table.append(blk)
            elif self.ref[table[-1]] > 1:
                blk = self._allocate()
                self.ref[blk] = 1
                self.copies.append((table[-1], blk, n % bs))
                self.ref[table[-1]] -= 1
                table[-1] = blk
            have.append(t)
            n += 1
            if n % bs == 0:
                self._register(table[-1], have, n)

    def fork(self, parent: int, child: int) -> None:
        assert child not in self.tables
        for b in self.tables[parent]:
            self.ref[b] += 1
        self.tables[child] = list(self.tables[parent])
        self.tokens[child] = list(self.tokens[parent])

    def release(self, seq: int) -> None:
        for b in reversed(self.tables.pop(seq)):
            self._release(b)
        del self.tokens[seq]

    def take_copies(self) -> List[Tuple[int, int, int]]:
        c, self.copies = self.copies, []
        return c

    # ------------------------------------------------------------ views
    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def num_free(self) -> int:
        return len(self.free)

    def num_evictable(self) -> int:
        return len(self.lru)
