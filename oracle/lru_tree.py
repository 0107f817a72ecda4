"""Plain radix tree with locks and LRU eviction: the model of the prefix cache
once memory runs short.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the native radix tree in ``prefix_shared_kv_amd`` and never imports it.

What the pages fix
------------------
SGLang summary (unite.ai), RadixAttention bullet: the runtime keeps an LRU
cache of KV in a radix tree and uses the tree to match, insert and evict.  The
nine-step example, steps 4-9: edges split where two sessions or few-shot
queries share part of them (4, 7); when memory runs short the least recently
used nodes are evicted (5: one node; 8: every node of the idle second session;
9: several nodes, to make room for parallel samples), never the nodes the
incoming requests reuse.

Eviction is a policy, not a closed form, so this model takes its steps as the
example describes them, written plainly (nodes are Python objects, candidates
are found by scanning the whole tree on every removal).  Readings where the
pages are silent:
  * a node is "used" by a call whose tokens enter its edge (at least one token
    matched); match and emit_rows use every node the request's tokens enter,
    one time for a whole batch; insert uses the nodes it passes through and its
    new leaf, and of an edge it splits only the upper part (the part it matched);
  * the unit of eviction is a whole node, and only a leaf: removing an inner
    node would orphan its children;
  * a running request pins the nodes holding its cached prefix: the deepest
    node its prefix enters (its whole edge, even when the prefix ends inside
    it) and every ancestor.  A pin is held as the token path it covers, so a
    later split of a pinned edge leaves both parts pinned;
  * among evictable leaves the least recently used goes first; equal times are
    broken by the lower first slot of the edge;
  * evicted slots return to the back of the free list in position order, and a
    parent left without children becomes a candidate in turn;
  * a batch that lacks free slots pins its matched prefixes, marks the nodes it
    enters as used, evicts what it lacks, then allocates as usual.
The radix bookkeeping itself (exact-prefix match capped at n-1, FIFO slots,
first writer wins) is that of ``radix_ref.RadixRef``, which pins this model
where nothing is evicted.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Optional, Sequence, Tuple

from .radix_ref import OutOfSlots


class _Node:
    def __init__(self, parent: Optional["_Node"], tokens: List[int], slots: List[int], last_use: int):
        self.parent = parent
        self.tokens = tokens
        self.slots = slots
        self.children: Dict[int, "_Node"] = {}
        self.last_use = last_use

    def path(self) -> Tuple[int, ...]:
        parts = []
        n = self
        while n is not None:
            parts.append(n.tokens)
            n = n.parent
        return tuple(t for p in reversed(parts) for t in p)


class LruTree:
    def __init__(self, pool_slots: int, free_order: Optional[Sequence[int]] = None):
        order = range(pool_slots) if free_order is None else [int(x) for x in free_order]
        self.free = deque(order)
        self.root = _Node(None, [], [], 0)
        self.time = 0
        self.pins: Dict[int, Tuple[int, ...]] = {}  # lock id -> pinned token path
        self._next_lock = 1
        self.splits = 0
        self.evicted_tokens = 0
        self.evicted_nodes = 0

    # -- tree walks ----------------------------------------------------------
    def _tick(self) -> int:
        self.time += 1
        return self.time

    def _enter(self, tokens: Sequence[int]) -> Tuple[List[Tuple[_Node, int]], int]:
        """The edges the tokens enter, each with the count of its tokens matched, and the matched length."""
        visits = []
        node, pos = self.root, 0
        while pos < len(tokens):
            child = node.children.get(tokens[pos])
            if child is None:
                break
            k = 0
            while k < len(child.tokens) and pos + k < len(tokens) and child.tokens[k] == tokens[pos + k]:
                k += 1
            visits.append((child, k))
            pos += k
            if k < len(child.tokens):
                break
            node = child
        return visits, pos

    def nodes(self) -> List[_Node]:
        out, stack = [], list(self.root.children.values())
        while stack:
            n = stack.pop()
            out.append(n)
            stack.extend(n.children.values())
        return out

    # -- cache operations ----------------------------------------------------
    def match(self, tokens: Sequence[int]) -> Tuple[int, List[int]]:
        tokens = [int(x) for x in tokens]
        visits, m = self._enter(tokens)
        now = self._tick()
        for node, _ in visits:
            node.last_use = now
        m = min(m, max(len(tokens) - 1, 0))
        slots = [s for node, k in visits for s in node.slots[:k]]
        return m, slots[:m]

    def alloc(self, n: int) -> List[int]:
        if n > len(self.free):
            raise OutOfSlots(n)
        return [self.free.popleft() for _ in range(n)]

    def free_slots(self, slots: Sequence[int]) -> None:
        self.free.extend(int(s) for s in slots)

    def _split(self, node: _Node, k: int) -> _Node:
        """The first k tokens of node's edge become a new parent node; node keeps the rest."""
        upper = _Node(node.parent, node.tokens[:k], node.slots[:k], node.last_use)
        node.parent.children[node.tokens[0]] = upper
        node.tokens, node.slots = node.tokens[k:], node.slots[k:]
        node.parent = upper
        upper.children[node.tokens[0]] = node
        self.splits += 1
        return upper

    def insert(self, tokens: Sequence[int], slots: Sequence[int]) -> Tuple[List[int], int]:
        """Store (tokens, slots); returns (the slots now backing tokens, number newly stored)."""
        tokens = [int(x) for x in tokens]
        slots = [int(s) for s in slots]
        assert len(tokens) == len(slots)
        now = self._tick()
        node, pos, stored = self.root, 0, 0
        while pos < len(tokens):
            child = node.children.get(tokens[pos])
            if child is None:
                node.children[tokens[pos]] = _Node(node, tokens[pos:], slots[pos:], now)
                stored = len(tokens) - pos
                break
            k = 0
            while k < len(child.tokens) and pos + k < len(tokens) and child.tokens[k] == tokens[pos + k]:
                k += 1
            for i in range(k):  # first writer wins: the caller's other slot goes back
                if slots[pos + i] != child.slots[i]:
                    self.free.append(slots[pos + i])
                    slots[pos + i] = child.slots[i]
            pos += k
            if k < len(child.tokens):
                if pos < len(tokens):
                    node = self._split(child, k)
                    node.last_use = now
                    continue
                child.last_use = now
                break
            child.last_use = now
            node = child
        return slots, stored

    # -- locks and eviction --------------------------------------------------
    def _pin(self, path: Tuple[int, ...]) -> int:
        lid = self._next_lock
        self._next_lock += 1
        self.pins[lid] = path
        return lid

    def lock(self, tokens: Sequence[int]) -> Tuple[int, int]:
        """Pin the cached prefix of tokens.  Returns (lock id, cached length)."""
        visits, m = self._enter([int(x) for x in tokens])
        return self._pin(visits[-1][0].path() if visits else ()), m

    def unlock(self, lock_id: int) -> None:
        del self.pins[lock_id]

    def pinned(self, node: _Node) -> bool:
        p = node.path()
        return any(len(q) >= len(p) and q[:len(p)] == p for q in self.pins.values())

    def evict(self, n_slots: int) -> int:
        freed = 0
        while freed < n_slots:
            leaves = [nd for nd in self.nodes() if not nd.children and not self.pinned(nd)]
            if not leaves:
                break
            victim = min(leaves, key=lambda nd: (nd.last_use, nd.slots[0]))
            del victim.parent.children[victim.tokens[0]]
            self.free.extend(victim.slots)
            freed += len(victim.tokens)
            self.evicted_tokens += len(victim.tokens)
            self.evicted_nodes += 1
        return freed

    def emit_rows(self, batch: Sequence[Sequence[int]], reserve: int = 0, evict: bool = False,
                  lock: bool = False):
        """Rows [prefix slots | new slots | reserved] for a batch.
        Returns (rows, prefix_lens, extend_lens, lock ids or None)."""
        batch = [[int(x) for x in t] for t in batch]
        walks = [self._enter(t) for t in batch]
        P = [min(m, max(len(t) - 1, 0)) for (_, m), t in zip(walks, batch)]
        need = sum(len(t) - p + reserve for t, p in zip(batch, P))
        short = need > len(self.free)
        if short and not evict:
            raise OutOfSlots(need)
        locks = []
        if lock or short:
            for (visits, _), p in zip(walks, P):
                deepest, w = None, 0
                for node, k in visits:
                    if w >= p:
                        break
                    deepest, w = node, w + k
                locks.append(self._pin(deepest.path() if deepest is not None else ()))
        now = self._tick()
        for visits, _ in walks:
            for node, _ in visits:
                node.last_use = now
        if short:
            self.evict(need - len(self.free))
            if need > len(self.free):
                for lid in locks:
                    self.unlock(lid)
                raise OutOfSlots(need)
        rows = []
        for (visits, _), t, p in zip(walks, batch, P):
            prefix = [s for node, k in visits for s in node.slots[:k]][:p]
            rows.append(prefix + self.alloc(len(t) - p + reserve))
        if not lock:
            for lid in locks:
                self.unlock(lid)
            locks = None
        return rows, P, [len(t) - p for t, p in zip(batch, P)], locks

    # -- observables -----------------------------------------------------------
    def stats(self) -> dict:
        ns = self.nodes()
        return {"nodes": len(ns), "cached_tokens": sum(len(n.tokens) for n in ns), "free_slots": len(self.free),
                "splits": self.splits, "evicted_tokens": self.evicted_tokens, "evicted_nodes": self.evicted_nodes,
                "locked_tokens": sum(len(n.tokens) for n in ns if self.pinned(n))}

    def sequences(self) -> List[Tuple[Tuple[int, ...], List[int]]]:
        """Every root-to-leaf path with its slots: what the cache holds."""
        out = []
        for n in self.nodes():
            if not n.children:
                slots, m = [], n
                while m is not None:
                    slots = m.slots + slots
                    m = m.parent
                out.append((n.path(), slots))
        return sorted(out)
