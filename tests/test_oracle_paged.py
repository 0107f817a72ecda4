"""Pins for the paged bookkeeping model (oracle/radix_ref.PagedRadixRef): at
page size 1 it is the token-level model; the glossary's GPT-2 example at page
size 16 (the numbers it prints, rounded to whole pages); hand-worked cases of
the page-boundary hit loss, the cap and first-writer-wins per page."""
import json
import os

import numpy as np
import pytest

from oracle.radix_ref import OutOfSlots, PagedRadixRef, RadixRef

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prompt_cache_gpt2_bookkeeping.json")


def _workload(seed, n=40):
    g = np.random.default_rng(seed)
    stems = [list(g.integers(0, 6, size=g.integers(1, 14))) for _ in range(4)]
    out = []
    for _ in range(n):
        s = stems[g.integers(0, len(stems))]
        cut = int(g.integers(0, len(s) + 1))
        out.append([int(x) for x in s[:cut]] + [int(x) for x in g.integers(0, 6, size=g.integers(1, 6))])
    return out


@pytest.mark.parametrize("seed", range(5))
def test_page_size_one_is_the_token_model(seed):
    reqs = _workload(seed)
    pr, tr = PagedRadixRef(2048, 1), RadixRef(2048)
    for i in range(0, len(reqs), 3):
        batch = reqs[i:i + 3]
        got = pr.emit_rows(batch, reserve=2)
        assert got == tr.emit_rows(batch, reserve=2)
        for r, row in zip(batch, got[0]):
            assert pr.insert(r, row[:len(r)]) == tr.insert(r, row[:len(r)])
        for r in batch:
            assert pr.match(r) == tr.match(r)
    assert list(pr.free) == list(tr.free)


def test_gpt2_example_at_page_size_16():
    # the glossary prefills a 409-token prompt, then runs questions of 8 and 7
    # tokens ("Computed 8 of 417", "7 of 416" at one token per slot).  With
    # 16-token pages only the 25 full pages (400 tokens) of the prompt are
    # stored, so each question also recomputes the prompt's last 9 tokens.
    g = json.load(open(GOLDEN))
    P, ps = g["prefix_tokens"], 16
    r = PagedRadixRef(256, ps)
    prefix = list(range(1000, 1000 + P))
    rows, plens, _ = r.emit_rows([prefix])
    assert plens == [0] and len(rows[0]) == (P + ps - 1) // ps
    canon, stored = r.insert(prefix, rows[0])
    assert stored == P // ps == 25
    for i, qd in enumerate(g["questions"]):
        q = [50000 + 100 * i + j for j in range(qd["new_tokens"])]
        n = P + len(q)
        assert n == qd["printed_total"]
        m, ids = r.match(prefix + q)
        assert m == (P // ps) * ps == 400 and ids == canon[:25]
        assert n - m == qd["new_tokens"] + P % ps  # 17 of 417, 16 of 416


def test_divergence_inside_a_page_shares_only_whole_pages():
    r = PagedRadixRef(64, 4)
    a = list(range(1, 11))          # 2 full pages + 2 tokens
    b = a[:10] + [77, 78, 79]       # same 10 tokens, then different
    c = a[:6] + [99] * 6            # diverges inside the second page
    rows, _, _ = r.emit_rows([a])
    r.insert(a, rows[0])
    assert r.match(b) == (8, rows[0][:2])        # the partial third page is not stored
    assert r.match(c) == (4, rows[0][:1])        # the second page differs: only the first is shared
    assert r.match(a[:4] + [5]) == (4, rows[0][:1])
    assert r.match(a[:3]) == (0, [])             # shorter than a page


def test_cap_keeps_one_token_when_every_page_is_cached():
    r = PagedRadixRef(64, 4)
    a = list(range(1, 13))  # exactly 3 pages
    rows, _, _ = r.emit_rows([a])
    r.insert(a, rows[0])
    assert r.match(a) == (8, rows[0][:2])        # the last page is computed again
    assert r.match(a + [5]) == (12, rows[0][:3])
    P_rows, P, E = r.emit_rows([a], reserve=2)
    assert P == [8] and E == [4] and len(P_rows[0]) == 2 + 2  # 12 + 2 tokens -> 4 pages


def test_first_writer_wins_per_page_and_all_or_nothing():
    r = PagedRadixRef(10, 2, free_order=[9, 8, 7, 6, 5, 4, 3, 2, 1, 0])
    x = [1, 2, 3, 4, 5]
    rows, _, _ = r.emit_rows([x, x])               # both miss: 3 pages each
    assert rows == [[9, 8, 7], [6, 5, 4]]
    r.insert(x, rows[0])
    canon, stored = r.insert(x, rows[1])            # the second copy's 2 full pages are freed
    assert canon == [9, 8] and stored == 0 and list(r.free)[-2:] == [6, 5]
    with pytest.raises(OutOfSlots):
        r.emit_rows([[1] * 9, [2] * 9])             # 5 + 5 pages, 6 free
    assert len(r.free) == 6
