"""Plain model of the host-memory prefix cache's policy (test infrastructure).

TEST INFRASTRUCTURE: only the test suite and the benchmark's CPU leg use it.

What it models [9c1h.cn news page, section "秘訣2"; explinks.com page
"Character.AI 的最佳实践", sections "有状态缓存" and "LRU 缓存结构"]: the KV of
conversation prefixes is cached between turns in a tree with least-recently-
used eviction; a request gets the longest cached prefix, partial matches
included. Reading used (the pages give no more): the unit is a block of
``block_size`` tokens; a cached block stands for the exact token prefix that
ends with it; the longest match is the longest run of cached block prefixes
from the start; eviction removes the least recently used block that no
cached block extends; a match or an insert uses every block of its chain,
oldest first; an insert stops when the only evictable block is the end of
the chain it is extending.

Here a cached block is literally its token tuple (no hashing, no slots), so
the model can be checked by eye.
"""
from __future__ import annotations


class PrefixCacheRef:
    def __init__(self, block_size: int, capacity_blocks: int):
        self.bs = int(block_size)
        self.cap = int(capacity_blocks)
        self.last_use: dict[tuple, int] = {}
        self.clock = 0
        self.evicted = 0

    def _touch(self, key: tuple) -> None:
        self.clock += 1
        self.last_use[key] = self.clock

    def _is_leaf(self, key: tuple) -> bool:
        n = len(key) + self.bs
        return not any(len(k) == n and k[: len(key)] == key for k in self.last_use)

    def _chain(self, tokens) -> list[tuple]:
        chain = []
        for k in range(1, len(tokens) // self.bs + 1):
            key = tuple(tokens[: k * self.bs])
            if key not in self.last_use:
                break
            chain.append(key)
        return chain

    def match(self, tokens) -> int:
        chain = self._chain(tokens)
        for key in chain:
            self._touch(key)
        return len(chain) * self.bs

    def insert(self, tokens) -> tuple[int, int]:
        """Returns (first_new_block, n_blocks) as the library does."""
        chain = self._chain(tokens)
        for key in chain:
            self._touch(key)
        first_new = len(chain)
        parent = chain[-1] if chain else None
        done = first_new
        for k in range(first_new, len(tokens) // self.bs):
            if len(self.last_use) >= self.cap:
                leaves = [key for key in self.last_use if self._is_leaf(key)]
                victim = min(leaves, key=lambda key: self.last_use[key])
                if victim == parent:
                    break
                del self.last_use[victim]
                self.evicted += 1
            key = tuple(tokens[: (k + 1) * self.bs])
            self._touch(key)
            parent = key
            done = k + 1
        return first_new, done

    def cached_blocks(self) -> int:
        return len(self.last_use)
