"""Plain Python reference of the paged KV block manager (host side).

TEST INFRASTRUCTURE ONLY.  Only the tests and the CPU-baseline leg of the
benchmark may import or call this module.  The library's C++ block manager
never calls it and shares no code with it.

What it models, and where the pages describe it:

* MiniLLM Runtime ("Features" list; "Component graph"): KV block allocation,
  release, reuse and reference counting; per-request block tables; prefix
  cache lookup with shared block ownership.
* mini_engine ("Features", Serving): hash-based prefix caching in which a
  block gets its hash the moment it is full, which lets requests that are
  still part-way through their prefill share prefixes.
* miniserve ("Architecture": KVCacheManager with paged blocks, chained
  hashes, refcounts and an LRU free list; the request state diagram and the
  "Engine" flowchart): find_cached_prefix() matches whole blocks through
  chained block hashes and always leaves at least one token to compute;
  allocate() takes cached pages with refcount + 1 (reclaiming them from the
  free list) and pops new pages off the LRU front; freeing drops refcounts
  and appends pages that reach zero to the free-list tail, and their hashes
  stay reusable until the page is taken again; slot = block_id * block_size
  + offset.

Readings where the pages leave a step open (listed again in the design
notes): the free list starts as blocks 0 .. N-1 in order; a freed request's
pages go to the tail in block-table order; allocation is all-or-nothing; a
filled block whose content is already registered under another page keeps
that earlier registration; a page taken off the free list loses its
registration.  A cached block is identified by its whole token prefix, so
this reference keys its map by the exact prefix tuple (no hashing at all);
an implementation that hashes must reach the same hits.
"""

from __future__ import annotations

from collections import OrderedDict

__all__ = ["RefBlockManager"]


class _Req:
    __slots__ = ("tokens", "blocks", "computed")

    def __init__(self, tokens):
        self.tokens = list(tokens)
        self.blocks: list[int] = []
        self.computed = 0


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self.B = block_size
        self.N = num_blocks
        self.refcount = [0] * num_blocks
        self.free: OrderedDict[int, None] = OrderedDict((b, None) for b in range(num_blocks))
        self.prefix_to_block: dict[tuple, int] = {}
        self.block_prefix: dict[int, tuple] = {}
        self.reqs: dict[int, _Req] = {}

    # -- requests -------------------------------------------------------
    def add_request(self, rid: int, prompt) -> None:
        if rid in self.reqs:
            raise KeyError(f"request {rid} exists")
        self.reqs[rid] = _Req(prompt)

    def append_token(self, rid: int, token: int) -> None:
        self.reqs[rid].tokens.append(int(token))

    def num_free(self) -> int:
        return len(self.free)

    def _blocks_for(self, ntok: int) -> int:
        return -(-ntok // self.B)

    # -- prefix cache -----------------------------------------------------
    def find_cached_prefix(self, rid: int) -> list[int]:
        """Pages holding the request's longest cached whole-block prefix,
        leaving at least one token to compute."""
        toks = self.reqs[rid].tokens
        hits = []
        for j in range(len(toks) // self.B):
            b = self.prefix_to_block.get(tuple(toks[:(j + 1) * self.B]))
            if b is None:
                break
            hits.append(b)
        if hits and len(hits) * self.B >= len(toks):
            hits.pop()
        return hits

    def _take_free(self, b: int) -> None:
        del self.free[b]

    def _pop_new(self) -> int:
        b, _ = self.free.popitem(last=False)  # LRU front
        key = self.block_prefix.pop(b, None)
        if key is not None and self.prefix_to_block.get(key) == b:
            del self.prefix_to_block[key]  # the page is taken: its content is gone
        return b

    # -- allocation -----------------------------------------------------
    def admit(self, rid: int, first_chunk: int) -> int | None:
        """find_cached_prefix + allocate(first_chunk) as one all-or-nothing
        step.  Returns the number of cached tokens, or None when the pool
        cannot hold the request's next first_chunk tokens."""
        r = self.reqs[rid]
        if r.blocks:
            raise ValueError("request already holds pages")
        hits = self.find_cached_prefix(rid)
        cached = len(hits) * self.B
        reclaimed = sum(1 for b in hits if self.refcount[b] == 0)
        new = self._blocks_for(cached + first_chunk) - len(hits)
        if new > len(self.free) - reclaimed:
            return None
        for b in hits:
            if self.refcount[b] == 0:
                self._take_free(b)
            self.refcount[b] += 1
        r.blocks = list(hits)
        r.computed = cached
        for _ in range(max(new, 0)):
            b = self._pop_new()
            self.refcount[b] = 1
            r.blocks.append(b)
        return cached

    def allocate(self, rid: int, n: int) -> bool:
        """Room for the next n tokens of a running request (all or nothing)."""
        r = self.reqs[rid]
        new = self._blocks_for(r.computed + n) - len(r.blocks)
        if new > len(self.free):
            return False
        for _ in range(max(new, 0)):
            b = self._pop_new()
            self.refcount[b] = 1
            r.blocks.append(b)
        return True

    def commit(self, rid: int, n: int) -> None:
        """n more tokens now have K/V in the cache; every block this fills is
        registered under its token prefix (unless that prefix already is)."""
        r = self.reqs[rid]
        before = r.computed // self.B
        r.computed += n
        if r.computed > len(r.tokens) or r.computed > len(r.blocks) * self.B:
            raise ValueError("commit past the known tokens or the allocated pages")
        for j in range(before, r.computed // self.B):
            key = tuple(r.tokens[:(j + 1) * self.B])
            b = r.blocks[j]
            if key not in self.prefix_to_block and b not in self.block_prefix:
                self.prefix_to_block[key] = b
                self.block_prefix[b] = key

    def free_request(self, rid: int, drop: bool = True) -> None:
        """Release the request's pages (refcount - 1, zero -> free-list tail,
        registrations kept).  drop=False keeps the request (preemption:
        nothing computed any more, tokens kept)."""
        r = self.reqs[rid]
        for b in r.blocks:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free[b] = None
        r.blocks = []
        r.computed = 0
        if drop:
            del self.reqs[rid]

    # -- views ------------------------------------------------------------
    def block_table(self, rid: int) -> list[int]:
        return list(self.reqs[rid].blocks)

    def slot_mapping(self, rid: int, start: int, n: int) -> list[int]:
        r = self.reqs[rid]
        return [r.blocks[p // self.B] * self.B + p % self.B for p in range(start, start + n)]

    def computed(self, rid: int) -> int:
        return self.reqs[rid].computed
