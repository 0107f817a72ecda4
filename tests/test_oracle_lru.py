"""Pins for the LRU radix-tree model (oracle/lru_tree.py): the nine-step
example of the SGLang summary, agreement with the tree-free brute-force model
wherever nothing is evicted, and the closed cases of LRU eviction."""
import json
import os

import numpy as np
import pytest

from oracle.lru_tree import LruTree
from oracle.radix_ref import OutOfSlots, RadixRef

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sglang_nine_step_lru.json")


def nine_steps():
    return json.load(open(GOLDEN))


def seq_of(fx, names):
    return tuple(t for n in names for t in fx["segments"][n])


def test_nine_step_example():
    fx = nine_steps()
    t = LruTree(fx["pool_slots"])
    for st in fx["steps"]:
        reqs = [list(seq_of(fx, r)) for r in st["requests"]]
        ev0 = (t.evicted_nodes, t.evicted_tokens)
        rows, P, E, locks = t.emit_rows(reqs, reserve=st["reserve"], evict=True, lock=True)
        assert P == st["prefix_lens"], st["step"]
        assert (t.evicted_nodes - ev0[0], t.evicted_tokens - ev0[1]) == (st["evicted_nodes"], st["evicted_tokens"]), st["step"]
        if st["commit"]:
            for r, row in zip(reqs, rows):
                t.insert(r, row[:len(r)])
        for lid in locks:
            t.unlock(lid)
        for r, row, p in zip(reqs, rows, P):
            t.free_slots(row[len(r):] if st["commit"] else row[p:])
        assert [s for s, _ in t.sequences()] == sorted(seq_of(fx, c) for c in st["cached"]), st["step"]
        assert t.stats()["nodes"] == st["nodes"], st["step"]
        # every slot is either cached or free, once
        held = [s for n in t.nodes() for s in n.slots]
        assert sorted(held + list(t.free)) == list(range(fx["pool_slots"])), st["step"]


def _workload(seed, n_req=40):
    """Requests over a few shared prefixes with random continuations."""
    g = np.random.default_rng(seed)
    stems = [list(g.integers(0, 50, size=g.integers(1, 12))) for _ in range(5)]
    out = []
    for _ in range(n_req):
        s = list(stems[g.integers(0, len(stems))])
        cut = int(g.integers(0, len(s) + 1))
        out.append([int(x) for x in s[:cut]] + [int(x) for x in g.integers(0, 50, size=g.integers(1, 8))])
    return out


@pytest.mark.parametrize("seed", range(6))
def test_without_eviction_equals_the_bruteforce_model(seed):
    # RadixRef keeps no tree: it answers from the list of stored sequences
    reqs = _workload(seed)
    tree, ref = LruTree(4096), RadixRef(4096)
    for i in range(0, len(reqs), 4):
        batch = reqs[i:i + 4]
        rows_t, P_t, E_t, _ = tree.emit_rows(batch, reserve=2)
        rows_r, P_r, E_r = ref.emit_rows(batch, reserve=2)
        assert (rows_t, P_t, E_t) == (rows_r, P_r, E_r)
        for r, row in zip(batch, rows_t):
            assert tree.insert(r, row[:len(r)]) == ref.insert(r, row[:len(r)])
        for r in batch:
            assert tree.match(r) == ref.match(r)
    assert list(tree.free) == list(ref.free)


def test_lru_order_of_independent_sequences():
    # textbook LRU: disjoint sequences leave in the order of their last use
    t = LruTree(64)
    seqs = [[100 * i + j for j in range(3)] for i in range(1, 6)]
    for s in seqs:
        t.insert(s, t.alloc(3))
    for i in (2, 0, 4):  # refresh: order of last use is now 1, 3, 2, 0, 4
        t.match(seqs[i] + [9999])
    left = [tuple(s) for s in seqs]
    for i in (1, 3, 2, 0, 4):
        assert t.evict(1) == 3
        left.remove(tuple(seqs[i]))
        assert [s for s, _ in t.sequences()] == sorted(left)


def test_equal_times_go_by_first_slot():
    t = LruTree(16, free_order=[7, 8, 9, 1, 2, 3] + list(range(10, 16)) + [0, 4, 5, 6])
    a, b = [1, 2, 3], [4, 5, 6]
    t.insert(a, t.alloc(3))  # slots 7, 8, 9
    t.insert(b, t.alloc(3))  # slots 1, 2, 3
    t.emit_rows([a + [0], b + [0]])  # both used at the same time
    t.free_slots(list(range(10, 12)))
    assert t.evict(1) == 3
    assert [s for s, _ in t.sequences()] == [tuple(a)]  # b's edge starts at the lower slot


def test_evicting_everything_without_locks_empties_the_cache():
    t = LruTree(2048)
    for r in _workload(7):
        rows, P, E, _ = t.emit_rows([r])
        t.insert(r, rows[0])
    cached = t.stats()["cached_tokens"]
    assert t.evict(10 ** 9) == cached
    assert t.stats()["cached_tokens"] == 0 and t.stats()["nodes"] == 0
    assert sorted(t.free) == list(range(2048))


def test_locks_survive_full_eviction():
    t = LruTree(2048)
    reqs = _workload(8)
    for r in reqs:
        rows, _, _, _ = t.emit_rows([r])
        t.insert(r, rows[0])
    g = np.random.default_rng(8)
    held = []
    for i in g.choice(len(reqs), size=5, replace=False):
        n = int(g.integers(1, len(reqs[i]) + 1))
        lid, m = t.lock(reqs[i][:n])
        assert m == n
        held.append((lid, reqs[i][:n]))
    t.evict(10 ** 9)
    st = t.stats()
    assert st["cached_tokens"] == st["locked_tokens"] > 0
    for _, s in held:  # each locked prefix is still cached in full
        assert t.match(list(s) + [-1])[0] == len(s)
    for lid, _ in held:
        t.unlock(lid)
    t.evict(10 ** 9)
    assert t.stats()["cached_tokens"] == 0


def test_a_pinned_edge_split_later_stays_pinned():
    t = LruTree(64)
    t.insert(list(range(1, 11)), t.alloc(10))
    lid, m = t.lock([1, 2, 3, 4, 5])  # ends inside the edge: the whole edge is pinned
    assert m == 5
    t.insert([1, 2, 3, 20, 21], [0, 1, 2] + t.alloc(2))  # splits the pinned edge after 3 tokens
    assert t.stats()["splits"] == 1
    assert t.evict(10 ** 9) == 2  # only the unpinned branch can go
    assert [s for s, _ in t.sequences()] == [tuple(range(1, 11))]
    t.unlock(lid)
    assert t.evict(10 ** 9) == 10


def test_use_times_never_increase_downward():
    # a walk that uses a node uses its ancestors too, so a parent is never
    # less recently used than its child and eviction removes leaves first
    t = LruTree(96)  # small enough that batches evict
    reqs = _workload(9, 60)
    g = np.random.default_rng(9)
    for i in range(0, len(reqs), 3):
        batch = reqs[i:i + 3]
        rows, P, E, _ = t.emit_rows(batch, evict=True)
        for r, row, p in zip(batch, rows, P):
            if g.random() < 0.7:
                t.insert(r, row)
            else:
                t.free_slots(row[p:])
        t.match(reqs[int(g.integers(0, len(reqs)))])
        for n in t.nodes():
            if n.parent is not t.root:
                assert n.parent.last_use >= n.last_use
    assert t.evicted_nodes > 0


def test_short_batch_evicts_only_what_it_lacks_and_keeps_its_prefix():
    t = LruTree(20)
    a = list(range(1, 9))
    b = list(range(21, 29))
    t.insert(a, t.alloc(8))
    t.insert(b, t.alloc(8))
    # 4 free; a request reusing a needs 6: b (not a) must go, and it is enough
    rows, P, E, locks = t.emit_rows([a + [90, 91, 92, 93, 94, 95]], evict=True, lock=True)
    assert P == [8] and t.evicted_nodes == 1
    assert [s for s, _ in t.sequences()] == [tuple(a)]
    assert t.stats()["locked_tokens"] == 8
    with pytest.raises(OutOfSlots):  # a is pinned: nothing left to evict
        t.emit_rows([[50] * 20], evict=True)
    assert t.stats()["locked_tokens"] == 8 and len(t.pins) == 1


def test_split_lower_part_keeps_its_last_use():
    # an insert that diverges inside an edge uses only the part it matched:
    # the lower part keeps its older time and leaves before the new branch,
    # although the new branch's edge starts at a lower slot
    t = LruTree(16, free_order=list(range(10, 16)) + list(range(10)))
    t.insert([1, 2, 3, 4, 5, 6], t.alloc(6))  # slots 10..15
    t.insert([1, 2, 9], [10, 11] + t.alloc(1))  # splits after [1, 2]; the new leaf [9] gets slot 0
    assert t.evict(1) == 4
    assert [s for s, _ in t.sequences()] == [(1, 2, 9)]
