"""Brute-force model of the prefix cache's observable bookkeeping.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the native radix tree in ``prefix_shared_kv_amd`` and never imports it.

What the pages fix
------------------
* "Prompt Caching" glossary (ultralytics), opening paragraph and the section on
  hosted APIs: reuse needs an *exactly* identical prefix; on a hit only the new
  tokens are processed.
* SGLang summary (unite.ai), RadixAttention bullet and the nine-step example:
  the runtime keeps KV in a radix tree and uses it for matching, inserting and
  evicting; a new turn reuses the cached prefix and is inserted as a new node;
  nodes are split when two sessions (or few-shot queries) share part of an edge.

This model keeps no tree at all: it stores every inserted (token sequence,
slot list) pair and answers a match with the longest common prefix over all of
them, which is what a radix tree computes, whatever its node boundaries are.
Slot bookkeeping (readings where the pages are silent):
  * the match is capped at n-1 tokens, so every request runs at least one token
    (the tutorial still runs one token over an already warm prefix);
  * slots are handed out first-in first-out from an initial free order
    (identity, or a given permutation); freed slots go to the back;
  * inserting a sequence whose prefix is already stored keeps the stored slots
    ("first writer wins"); the caller's slots for those positions, where they
    differ, are freed in ascending position order;
  * a batch allocation is all-or-nothing, in request order: each request's new
    tokens, then its reserved decode slots.
"""
from __future__ import annotations

from collections import deque
from typing import List, Optional, Sequence, Tuple


class OutOfSlots(Exception):
    pass


def _lcp(a: Sequence[int], b: Sequence[int]) -> int:
    n = min(len(a), len(b))
    i = 0
    while i < n and a[i] == b[i]:
        i += 1
    return i


class RadixRef:
    def __init__(self, pool_slots: int, free_order: Optional[Sequence[int]] = None):
        order = range(pool_slots) if free_order is None else [int(x) for x in free_order]
        self.free = deque(order)
        self.seqs: List[Tuple[Tuple[int, ...], List[int]]] = []

    # longest common prefix with any stored sequence, uncapped
    def _longest(self, tokens: Sequence[int]) -> Tuple[int, List[int]]:
        best, best_slots = 0, []
        t = [int(x) for x in tokens]
        for seq, slots in self.seqs:
            m = _lcp(seq, t)
            if m > best:
                best, best_slots = m, slots[:m]
        return best, best_slots

    def match(self, tokens: Sequence[int]) -> Tuple[int, List[int]]:
        m, slots = self._longest(tokens)
        cap = max(len(tokens) - 1, 0)
        m = min(m, cap)
        return m, slots[:m]

    def alloc(self, n: int) -> List[int]:
        if n > len(self.free):
            raise OutOfSlots(n)
        return [self.free.popleft() for _ in range(n)]

    def free_slots(self, slots: Sequence[int]) -> None:
        self.free.extend(int(s) for s in slots)

    def insert(self, tokens: Sequence[int], slots: Sequence[int]) -> Tuple[List[int], int]:
        """Store (tokens, slots).  Returns (canonical slot list, number of newly cached tokens)."""
        assert len(tokens) == len(slots)
        m, stored = self._longest(tokens)
        slots = [int(s) for s in slots]
        dups = [slots[i] for i in range(m) if slots[i] != stored[i]]
        canon = stored[:m] + slots[m:]
        self.free_slots(dups)
        if m < len(tokens):
            self.seqs.append((tuple(int(x) for x in tokens), canon))
        return canon, len(tokens) - m

    def emit_rows(self, batch: Sequence[Sequence[int]], reserve: int = 0):
        """Rows of the request->slot table for a batch: [prefix slots | new slots | reserved].
        Returns (rows, prefix_lens, extend_lens)."""
        matches = [self.match(t) for t in batch]
        need = sum(len(t) - m + reserve for t, (m, _) in zip(batch, matches))
        if need > len(self.free):
            raise OutOfSlots(need)
        rows, plens, elens = [], [], []
        for t, (m, pre) in zip(batch, matches):
            new = self.alloc(len(t) - m + reserve)
            rows.append(list(pre) + new)
            plens.append(m)
            elens.append(len(t) - m)
        return rows, plens, elens

    def num_free(self) -> int:
        return len(self.free)


class PagedRadixRef:
    """The same bookkeeping at page granularity ("Prompt Caching" glossary, the
    serving-engine paragraph: KV kept in fixed-size blocks, the blocks of the
    longest matching prefix reused).  Readings where the pages are silent:
      * only full pages are stored and shared: a prefix matches in whole pages,
        the tokens of a partly matching page are computed again (the hit lost
        at page boundaries);
      * the cap keeps at least one token computed: at most (n - 1) // page_size
        pages of an n-token request are reused;
      * a request gets pages for its n + reserve tokens: the matched ones, then
        fresh ones, first-in first-out, all or nothing in request order;
      * inserting keeps the stored page where a page is already stored (first
        writer wins) and frees the caller's, in ascending page order.
    Like RadixRef it keeps no tree: stored sequences of full pages, each page a
    tuple of token ids."""

    def __init__(self, n_pages: int, page_size: int, free_order: Optional[Sequence[int]] = None):
        self.ps = page_size
        order = range(n_pages) if free_order is None else [int(x) for x in free_order]
        self.free = deque(order)
        self.seqs: List[Tuple[Tuple[Tuple[int, ...], ...], List[int]]] = []

    def pages(self, tokens: Sequence[int]) -> Tuple[Tuple[int, ...], ...]:
        t = [int(x) for x in tokens]
        return tuple(tuple(t[i * self.ps:(i + 1) * self.ps]) for i in range(len(t) // self.ps))

    def _longest(self, pg) -> Tuple[int, List[int]]:
        best, ids = 0, []
        for seq, pids in self.seqs:
            m = _lcp(seq, pg)
            if m > best:
                best, ids = m, pids[:m]
        return best, ids

    def match(self, tokens: Sequence[int]) -> Tuple[int, List[int]]:
        """(matched tokens, their page ids)."""
        m, ids = self._longest(self.pages(tokens))
        cap = (len(tokens) - 1) // self.ps if len(tokens) else 0
        m = min(m, cap)
        return m * self.ps, ids[:m]

    def alloc(self, n: int) -> List[int]:
        if n > len(self.free):
            raise OutOfSlots(n)
        return [self.free.popleft() for _ in range(n)]

    def free_pages(self, pids: Sequence[int]) -> None:
        self.free.extend(int(p) for p in pids)

    def insert(self, tokens: Sequence[int], pids: Sequence[int]) -> Tuple[List[int], int]:
        """Store the full pages of tokens with page ids pids[0 : len(tokens) // page_size].
        Returns (the page ids now backing those pages, number of pages newly stored)."""
        pg = self.pages(tokens)
        pids = [int(p) for p in pids[:len(pg)]]
        m, stored = self._longest(pg)
        dups = [pids[i] for i in range(m) if pids[i] != stored[i]]
        canon = stored[:m] + pids[m:]
        self.free_pages(dups)
        if m < len(pg):
            self.seqs.append((pg, canon))
        return canon, len(pg) - m

    def emit_rows(self, batch: Sequence[Sequence[int]], reserve: int = 0):
        """Rows of page ids [matched | fresh] per request.  Returns (rows, prefix_lens, extend_lens) in tokens."""
        matches = [self.match(t) for t in batch]
        npg = [(len(t) + reserve + self.ps - 1) // self.ps for t in batch]
        need = sum(k - P // self.ps for k, (P, _) in zip(npg, matches))
        if need > len(self.free):
            raise OutOfSlots(need)
        rows, plens, elens = [], [], []
        for t, k, (P, ids) in zip(batch, npg, matches):
            rows.append(list(ids) + self.alloc(k - P // self.ps))
            plens.append(P)
            elens.append(len(t) - P)
        return rows, plens, elens
