"""Reference model of KV block management: reference-counted blocks, per-sequence block tables with
copy-on-write, a prefix cache over whole blocks with least-recently-used eviction, and the block copy.

TEST INFRASTRUCTURE ONLY (like the rest of oracle/): only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never does, and the two share no code.

What the pages fix: the inferd page keeps a block allocator beside a page table and lists prefix
sharing among its follow-up plans (repository layout, core/paged_cache; follow-up plans); the
lfm25-inference page has the engine own the KV pages and reuse them across conversation turns through
a radix tree ("Runtime Design").  The rules below are the plain reading of those words:
  * a block's reference count is the number of its holders: each sequence whose table lists it, and
    each cached prefix that maps to it; a block with count 0 is free;
  * token p of a sequence lives in slot table[p // 16] * 16 + p % 16;
  * a sequence never writes into a block another holder still reads: before new tokens go into a
    shared, partly filled last block, the sequence switches to a fresh copy of it (copy-on-write);
  * the prefix cache maps token prefixes of whole blocks to the blocks that hold them, matches the
    longest cached prefix, and evicts least recently used entries that have no cached extension and
    no holder but the cache.
Which free block a call takes is not fixed by anything; the model does not choose ids.  It takes
the ids the implementation reports and checks that they are valid (the block was free, distinct),
then derives everything that is unique (slots, counts, copies, matches, evictions) on its own.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16


class BlockModel:
    def __init__(self, num_blocks: int):
        self.num_blocks = num_blocks
        self.tables: Dict[int, List[int]] = {}     # sequence key -> block table
        self.lengths: Dict[int, int] = {}
        self.cache: Dict[Tuple[int, ...], Tuple[int, int]] = {}   # prefix -> (block, last use)
        self.clock = 0

    # ---- counts ----
    def refcount(self, b: int) -> int:
        held = sum(t.count(b) for t in self.tables.values())
        return held + sum(1 for blk, _ in self.cache.values() if blk == b)

    def free_blocks(self) -> List[int]:
        return [b for b in range(self.num_blocks) if self.refcount(b) == 0]

    # ---- sequences ----
    def new_seq(self, key: int) -> None:
        self.tables[key] = []
        self.lengths[key] = 0

    def drop_seq(self, key: int) -> None:
        del self.tables[key]
        del self.lengths[key]

    def fork(self, key: int, child: int) -> None:
        self.tables[child] = list(self.tables[key])
        self.lengths[child] = self.lengths[key]

    def adopt(self, key: int, blocks: Sequence[int]) -> None:
        assert self.lengths[key] == 0 and not self.tables[key]
        self.tables[key] = [int(b) for b in blocks]
        self.lengths[key] = BLOCK * len(blocks)

    def append_needs(self, key: int, n: int) -> Tuple[int, bool]:
        """(fresh blocks, whether the last block must be copied first) for n new tokens."""
        length, table = self.lengths[key], self.tables[key]
        fresh = -(-(length + n) // BLOCK) - len(table)
        cow = n > 0 and length % BLOCK != 0 and self.refcount(table[-1]) > 1
        return fresh, cow

    def step_needs(self, keys: Sequence[int], ns: Sequence[int]) -> int:
        """Blocks a step of appends needs when they are done one after another in the given order
        (an earlier copy can leave a later sharer the sole holder): counted on a scratch copy."""
        scratch = BlockModel(self.num_blocks)
        scratch.tables = {k: list(t) for k, t in self.tables.items()}
        scratch.lengths = dict(self.lengths)
        scratch.cache = dict(self.cache)
        total = 0
        for k, n in zip(keys, ns):
            fresh, cow = scratch.append_needs(k, n)
            total += fresh + cow
            free = scratch.free_blocks()
            if fresh + cow > len(free):
                return total
            t = list(scratch.tables[k])
            if cow:
                t[-1] = free[fresh]
            scratch.append(k, n, t + free[:fresh])
        return total

    def append(self, key: int, n: int, new_table: Sequence[int]) -> Tuple[np.ndarray, Optional[Tuple[int, int]]]:
        """Apply an append whose resulting table the implementation reports; check that table and
        return the expected slots and copy pair."""
        fresh, cow = self.append_needs(key, n)
        old = self.tables[key]
        new_table = [int(b) for b in new_table]
        free = set(self.free_blocks())
        assert len(new_table) == len(old) + fresh, "one new block per 16 tokens past the last block"
        taken = new_table[len(old):]
        copy = None
        if cow:
            assert new_table[:len(old) - 1] == old[:-1]
            taken = taken + [new_table[len(old) - 1]]
            copy = (old[-1], new_table[len(old) - 1])
        else:
            assert new_table[:len(old)] == old
        assert len(set(taken)) == len(taken) and set(taken) <= free, "new blocks were free and distinct"
        self.tables[key] = new_table
        start = self.lengths[key]
        self.lengths[key] = start + n
        pos = np.arange(start, start + n)
        slots = np.asarray([new_table[p // BLOCK] * BLOCK + p % BLOCK for p in pos], dtype=np.int64)
        return slots, copy

    # ---- prefix cache ----
    def match(self, tokens: Sequence[int]) -> List[int]:
        self.clock += 1
        out = []
        for j in range(len(tokens) // BLOCK):
            key = tuple(int(t) for t in tokens[:(j + 1) * BLOCK])
            if key not in self.cache:
                break
            blk, _ = self.cache[key]
            self.cache[key] = (blk, self.clock)
            out.append(blk)
        return out

    def insert(self, tokens: Sequence[int], blocks: Sequence[int]) -> int:
        self.clock += 1
        added = 0
        for j in range(len(tokens) // BLOCK):
            key = tuple(int(t) for t in tokens[:(j + 1) * BLOCK])
            blk = self.cache[key][0] if key in self.cache else int(blocks[j])
            added += key not in self.cache
            self.cache[key] = (blk, self.clock)
        return added

    def _has_extension(self, key) -> bool:
        return any(len(k) == len(key) + BLOCK and k[:len(key)] == key for k in self.cache)

    def evict(self, n: int) -> int:
        freed = 0
        while freed < n:
            cands = [(used, key) for key, (blk, used) in self.cache.items()
                     if not self._has_extension(key) and self.refcount(blk) == 1]
            if not cands:
                break
            cands.sort()
            assert len(cands) == 1 or cands[0][0] != cands[1][0], "least recently used entry is unique"
            del self.cache[cands[0][1]]
            freed += 1
        return freed


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, src: Sequence[int], dst: Sequence[int]):
    """Pools after block dst[k] of each becomes a copy of block src[k] (ids outside the pool skipped)."""
    k2, v2 = k_cache.copy(), v_cache.copy()
    nb = k_cache.shape[0]
    for s, d in zip(src, dst):
        if 0 <= s < nb and 0 <= d < nb:
            k2[d] = k_cache[s]
            v2[d] = v_cache[s]
    return k2, v2
