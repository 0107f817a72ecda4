"""Locks and LRU eviction of the C++ radix tree against the plain model in
oracle/lru_tree.py: on the nine-step example and on random operation streams
(batches that evict and lock, commits, releases, explicit evictions) the
prefix lengths, table rows, free-list order and the tree's counters must
agree exactly."""
import json
import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle.lru_tree import LruTree
from oracle.radix_ref import OutOfSlots
from prefix_shared_kv_amd import RadixTree, RcError
from prefix_shared_kv_amd import _native as N

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sglang_nine_step_lru.json")
COUNTERS = ("nodes", "cached_tokens", "free_slots", "splits", "evicted_tokens", "evicted_nodes", "locked_tokens")


def same_state(tree: RadixTree, ref: LruTree):
    got = tree.stats()
    want = ref.stats()
    assert {k: got[k] for k in COUNTERS} == want


def test_nine_step_example_native():
    fx = json.load(open(GOLDEN))
    seg = fx["segments"]
    tree = RadixTree(fx["pool_slots"])
    table = np.full((4, 64), -1, np.int32)
    for stp in fx["steps"]:
        reqs = [[t for n in r for t in seg[n]] for r in stp["requests"]]
        B = len(reqs)
        before = tree.stats()
        h = np.zeros(B, np.int64)
        P, E = tree.emit_rows(reqs, table, reserve=stp["reserve"], evict=True, handles=h)
        assert P.tolist() == stp["prefix_lens"], stp["step"]
        after = tree.stats()
        assert after["evicted_nodes"] - before["evicted_nodes"] == stp["evicted_nodes"], stp["step"]
        assert after["evicted_tokens"] - before["evicted_tokens"] == stp["evicted_tokens"], stp["step"]
        if stp["commit"]:
            tree.insert_rows(reqs, table, np.arange(B, dtype=np.int32))
        tree.unlock(h)
        tails = [table[b, (len(r) if stp["commit"] else P[b]):len(r) + stp["reserve"]] for b, r in enumerate(reqs)]
        tree.free(np.concatenate(tails))
        st_ = tree.stats()
        assert st_["nodes"] == stp["nodes"], stp["step"]
        cached = [[t for n in c for t in seg[n]] for c in stp["cached"]]
        # every expected path is cached in full (lock reports the cached length
        # without marking nodes as used, which would change the LRU order) ...
        h2, m2 = tree.lock(cached)
        tree.unlock(h2)
        assert m2.tolist() == [len(c) for c in cached], stp["step"]
        # ... and nothing else (the tokens of the union of the paths)
        prefixes = {tuple(c[:i]) for c in cached for i in range(1, len(c) + 1)}
        assert st_["cached_tokens"] == len(prefixes), stp["step"]
        assert st_["free_slots"] + st_["cached_tokens"] == fx["pool_slots"], stp["step"]
        assert st_["locked_tokens"] == 0


def _seq(draw, base, vocab):
    stem = draw(st.sampled_from(base))
    tail = draw(st.lists(st.integers(0, vocab - 1), min_size=1, max_size=8))
    return stem[:draw(st.integers(0, len(stem)))] + tail


@st.composite
def streams(draw):
    vocab = draw(st.sampled_from([4, 50]))
    base = [draw(st.lists(st.integers(0, vocab - 1), min_size=1, max_size=14)) for _ in range(4)]
    ops = []
    for _ in range(draw(st.integers(1, 30))):
        kind = draw(st.sampled_from(["batch", "batch", "batch", "release", "evict", "match", "lock"]))
        if kind == "batch":
            ops.append((kind, [_seq(draw, base, vocab) for _ in range(draw(st.integers(1, 3)))],
                        draw(st.integers(0, 3)), draw(st.booleans()), draw(st.booleans())))
        elif kind == "evict":
            ops.append((kind, draw(st.integers(0, 40))))
        elif kind == "match":
            ops.append((kind, _seq(draw, base, vocab)))
        elif kind == "lock":
            ops.append((kind, _seq(draw, base, vocab), draw(st.integers(0, 20))))
        else:
            ops.append((kind, draw(st.integers(0, 10))))
    return ops, draw(st.sampled_from([48, 96, 160]))


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(streams())
def test_locks_and_eviction_match_the_model(sc):
    ops, S = sc
    order = np.random.default_rng(S).permutation(S).astype(np.int32)
    tree, ref = RadixTree(S, order), LruTree(S, order)
    table = np.full((3, 64), -1, np.int32)
    running = []  # (tokens, row slots, committed, native handles, model lock ids, P)
    held = []     # stand-alone locks: (native handle, model lock id)
    for op in ops:
        if op[0] == "batch":
            _, batch, reserve, commit, evict = op
            try:
                rows, P, E, lids = ref.emit_rows(batch, reserve=reserve, evict=evict, lock=True)
                ok = True
            except OutOfSlots:
                ok = False
            h = np.zeros(len(batch), np.int64)
            if ok:
                Pn, En = tree.emit_rows(batch, table, reserve=reserve, evict=evict, handles=h)
                assert Pn.tolist() == P and En.tolist() == E
                for b, r in enumerate(rows):
                    assert table[b, :len(r)].tolist() == r
                if commit:
                    for b, t in enumerate(batch):
                        rows[b][:len(t)] = ref.insert(t, rows[b][:len(t)])[0]
                    tree.insert_rows(batch, table, np.arange(len(batch), dtype=np.int32))
                    for b, r in enumerate(rows):
                        assert table[b, :len(r)].tolist() == r
                running.append((batch, rows, commit, h, lids, P))
            else:
                with pytest.raises(RcError) as e:
                    tree.emit_rows(batch, table, reserve=reserve, evict=evict, handles=h)
                assert e.value.status == N.RC_ERR_NOMEM
        elif op[0] == "release" and running:
            batch, rows, commit, h, lids, P = running.pop(op[1] % len(running))
            tree.unlock(h)
            for lid in lids:
                ref.unlock(lid)
            tails = [r[(len(t) if commit else p):] for t, r, p in zip(batch, rows, P)]
            flat = [s for tl in tails for s in tl]
            ref.free_slots(flat)
            tree.free(np.array(flat, np.int32))
        elif op[0] == "evict":
            assert tree.evict(op[1]) == ref.evict(op[1])
        elif op[0] == "match":
            m, s = tree.match(op[1])
            assert (m, s.tolist()) == ref.match(op[1])
        elif op[0] == "lock":
            t = op[1][:op[2]]
            hn, mn = tree.lock([t])
            lid, m = ref.lock(t)
            assert mn[0] == m
            held.append((hn, lid))
        same_state(tree, ref)
    for batch, rows, commit, h, lids, P in running:
        tree.unlock(h)
        for lid in lids:
            ref.unlock(lid)
    for hn, lid in held:
        tree.unlock(hn)
        ref.unlock(lid)
    assert tree.stats()["locked_tokens"] == 0
    assert tree.evict(10 ** 9) == ref.evict(10 ** 9)
    same_state(tree, ref)
    # the free lists hold the same slots in the same order
    n = tree.stats()["free_slots"]
    assert tree.alloc(n).tolist() == ref.alloc(n)


def test_unlock_rejects_bad_handles_and_changes_nothing():
    tree = RadixTree(32)
    tree.insert([1, 2, 3, 4], tree.alloc(4))
    h, m = tree.lock([[1, 2, 3, 4]])
    assert m.tolist() == [4] and h[0] != 0
    with pytest.raises(RcError):
        tree.unlock([h[0], h[0]])  # more releases than locks: nothing released
    assert tree.stats()["locked_tokens"] == 4
    with pytest.raises(RcError):
        tree.unlock([h[0] + (1 << 32)])  # wrong generation
    with pytest.raises(RcError):
        tree.unlock([12345])
    tree.unlock(h)
    assert tree.stats()["locked_tokens"] == 0
    tree.unlock([0])  # nothing pinned: a no-op
    # an evicted node's old handle is refused even after its id is reused
    assert tree.evict(100) == 4
    tree.insert([7, 8], tree.alloc(2))
    with pytest.raises(RcError):
        tree.unlock(h)


def test_lock_of_uncached_tokens_pins_nothing():
    tree = RadixTree(16)
    h, m = tree.lock([[5, 6, 7], []])
    assert h.tolist() == [0, 0] and m.tolist() == [0, 0]
    tree.unlock(h)


def test_emit_rows_without_evict_is_atomic_when_short():
    tree = RadixTree(10)
    tree.insert([1, 2, 3, 4, 5, 6], tree.alloc(6))
    table = np.full((1, 16), -1, np.int32)
    before = tree.stats()
    with pytest.raises(RcError) as e:
        tree.emit_rows([[9] * 6], table)
    assert e.value.status == N.RC_ERR_NOMEM
    assert tree.stats() == before and (table == -1).all()
    P, E = tree.emit_rows([[9] * 6], table, evict=True)
    assert (P.tolist(), E.tolist()) == ([0], [6]) and tree.stats()["evicted_tokens"] == 6
