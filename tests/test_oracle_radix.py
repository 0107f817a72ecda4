"""Pins for the brute-force prefix-cache model: the bookkeeping values the
glossary prints, and small hand-worked cases of exact-prefix reuse."""
import json
import os

import pytest

from oracle.radix_ref import OutOfSlots, RadixRef

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prompt_cache_gpt2_bookkeeping.json")


def test_gpt2_example_bookkeeping_values():
    g = json.load(open(GOLDEN))
    P = g["prefix_tokens"]
    ref = RadixRef(2048)
    prefix = list(range(1000, 1000 + P))
    # the prefill: a miss, every prefix token computed
    m, _ = ref.match(prefix)
    assert m == 0
    slots = ref.alloc(P)
    ref.insert(prefix, slots)
    for i, qd in enumerate(g["questions"]):
        q = [50000 + 100 * i + j for j in range(qd["new_tokens"])]
        m, pre = ref.match(prefix + q)
        computed = len(prefix + q) - m
        assert (computed, len(prefix + q)) == (qd["new_tokens"], qd["printed_total"])
        assert pre == slots  # the cached slots are the prefill's
        assert computed / len(prefix + q) < 0.02


def test_match_is_exact_prefix_only_and_capped():
    ref = RadixRef(64)
    s = ref.alloc(4)
    assert s == [0, 1, 2, 3]
    ref.insert([1, 2, 3, 4], s)
    assert ref.match([1, 2, 9]) == (2, [0, 1])
    assert ref.match([9, 2, 3]) == (0, [])
    assert ref.match([1, 2, 3, 4, 5]) == (4, [0, 1, 2, 3])
    # whole sequence cached: one token is still run
    assert ref.match([1, 2, 3, 4]) == (3, [0, 1, 2])
    assert ref.match([1]) == (0, [])
    assert ref.match([]) == (0, [])


def test_fifo_allocation_and_free_order():
    ref = RadixRef(6, free_order=[5, 3, 1, 0, 2, 4])
    assert ref.alloc(2) == [5, 3]
    ref.free_slots([3])
    assert ref.alloc(4) == [1, 0, 2, 4]
    assert ref.alloc(1) == [3]
    with pytest.raises(OutOfSlots):
        ref.alloc(1)


def test_insert_first_writer_wins_and_frees_duplicates():
    ref = RadixRef(16)
    a = ref.alloc(3)  # 0,1,2
    ref.insert([7, 8, 9], a)
    b = ref.alloc(4)  # 3,4,5,6 : same first two tokens computed again
    canon, n_new = ref.insert([7, 8, 5, 6], b)
    assert canon == [0, 1, 5, 6]
    assert n_new == 2
    # slots 3 and 4 went back to the end of the free list
    assert list(ref.free)[-2:] == [3, 4]
    # a sequence already fully present stores nothing and frees all its copies
    c = ref.alloc(2)
    canon, n_new = ref.insert([7, 8], c)
    assert canon == [0, 1] and n_new == 0
    assert list(ref.free)[-2:] == c


def test_emit_rows_all_or_nothing():
    ref = RadixRef(10)
    s = ref.alloc(4)
    ref.insert([1, 2, 3, 4], s)
    rows, P, E = ref.emit_rows([[1, 2, 3, 4, 5], [1, 2, 7]], reserve=1)
    assert P == [4, 2] and E == [1, 1]
    assert rows == [[0, 1, 2, 3, 4, 5], [0, 1, 6, 7]]
    free_before = list(ref.free)
    with pytest.raises(OutOfSlots):
        ref.emit_rows([[1, 9, 9, 9], [1, 2, 3, 4, 5]], reserve=0)
    assert list(ref.free) == free_before
