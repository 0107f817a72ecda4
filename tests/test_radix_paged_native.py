"""The C++ radix tree at page granularity (rc_radix_create_paged) against the
paged brute-force model (oracle/radix_ref.PagedRadixRef): prefix lengths, rows
of page ids, matches and the free list must agree exactly on random operation
streams; decode and cascade-extend plans from a paged tree must satisfy their
definition on the per-position slots the page rows stand for."""
import json
import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle.radix_ref import OutOfSlots, PagedRadixRef
from prefix_shared_kv_amd import RadixTree, RcError
from prefix_shared_kv_amd import _native as N

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prompt_cache_gpt2_bookkeeping.json")


def _seq(draw, base, vocab):
    stem = draw(st.sampled_from(base))
    tail = draw(st.lists(st.integers(0, vocab - 1), min_size=1, max_size=12))
    return stem[:draw(st.integers(0, len(stem)))] + tail


@st.composite
def streams(draw):
    vocab = draw(st.sampled_from([3, 50]))
    base = [draw(st.lists(st.integers(0, vocab - 1), min_size=1, max_size=24)) for _ in range(3)]
    ops = []
    for _ in range(draw(st.integers(1, 20))):
        kind = draw(st.sampled_from(["batch", "batch", "release", "match"]))
        if kind == "batch":
            ops.append((kind, [_seq(draw, base, vocab) for _ in range(draw(st.integers(1, 3)))],
                        draw(st.integers(0, 5)), draw(st.booleans())))
        elif kind == "match":
            ops.append((kind, _seq(draw, base, vocab)))
        else:
            ops.append((kind, draw(st.integers(0, 9))))
    return ops, draw(st.sampled_from([2, 4, 16])), draw(st.booleans())


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(streams())
def test_paged_tree_matches_the_model(sc):
    ops, ps, perm = sc
    n_pages = 48
    order = np.random.default_rng(ps).permutation(n_pages).astype(np.int32) if perm else None
    tree, ref = RadixTree(n_pages, order, page_size=ps), PagedRadixRef(n_pages, ps, order)
    table = np.full((3, 64), -1, np.int32)  # wide enough for any request of the stream
    running = []  # (tokens, model rows, committed)
    for op in ops:
        if op[0] == "batch":
            _, batch, reserve, commit = op
            try:
                rows, P, E = ref.emit_rows(batch, reserve=reserve)
            except OutOfSlots:
                with pytest.raises(RcError) as e:
                    tree.emit_rows(batch, table, reserve=reserve)
                assert e.value.status == N.RC_ERR_NOMEM
                continue
            entries = np.zeros(len(batch), np.int64)
            new_slots = np.full(sum(len(t) for t in batch) + 1, -7, np.int32)
            Pn, En = tree.emit_rows(batch, table, reserve=reserve, row_entries=entries, new_slots=new_slots)
            assert Pn.tolist() == P and En.tolist() == E
            o = 0
            for b, r in enumerate(rows):
                assert table[b, :len(r)].tolist() == r
                assert entries[b] == len(r)
                # new token at position p: slot = page(p // page_size) * page_size + p % page_size
                want = [r[p // ps] * ps + p % ps for p in range(P[b], P[b] + E[b])]
                assert new_slots[o:o + E[b]].tolist() == want
                o += E[b]
            assert (new_slots[o:] == -7).all()
            if commit:
                for b, t in enumerate(batch):
                    canon, _ = ref.insert(t, rows[b])
                    rows[b][:len(canon)] = canon
                tree.insert_rows(batch, table, np.arange(len(batch), dtype=np.int32))
                for b, r in enumerate(rows):
                    assert table[b, :len(r)].tolist() == r
            running.append((batch, rows, commit, P, table[:len(batch)].copy(), entries))
        elif op[0] == "release" and running:
            batch, rows, commit, P, tab, entries = running.pop(op[1] % len(running))
            own = []
            for t, r, p in zip(batch, rows, P):
                own += r[(len(t) // ps if commit else p // ps):]  # pages the tree does not hold
            ref.free_pages(own)
            keep = [len(t) for t in batch] if commit else P
            tree.free_rows(np.arange(len(batch)), tab, keep, entries)
        elif op[0] == "match":
            m, ids = tree.match(op[1])
            assert (m, ids.tolist()) == ref.match(op[1])
        st_ = tree.stats()
        assert st_["free_slots"] == len(ref.free)
        assert 0 < st_["page_symbols"] <= st_["cached_tokens"] or st_["page_symbols"] == st_["cached_tokens"] == 0
    n = len(ref.free)
    assert tree.alloc(n).tolist() == ref.alloc(n)
    # nothing is locked: eviction empties the tree and its page dictionary
    tree.evict(10 ** 6)
    assert tree.stats()["cached_tokens"] == 0 and tree.stats()["page_symbols"] == 0


def test_gpt2_example_at_page_size_16_native():
    g = json.load(open(GOLDEN))
    P, ps = g["prefix_tokens"], 16
    t = RadixTree(256, page_size=ps)
    prefix = np.arange(1000, 1000 + P, dtype=np.int32)
    table = np.full((2, 64), -1, np.int32)
    Pl, El = t.emit_rows([prefix], table)
    assert (Pl.tolist(), El.tolist()) == ([0], [P])
    t.insert_rows([prefix], table, [0])
    assert t.stats()["cached_tokens"] == P // ps  # pages
    for i, qd in enumerate(g["questions"]):
        q = np.arange(qd["new_tokens"], dtype=np.int32) + 50000 + 100 * i
        Pl, El = t.emit_rows([np.concatenate([prefix, q])], table, rows=[1])
        assert Pl[0] == 400 and El[0] == qd["new_tokens"] + P % ps  # 17 of 417, 16 of 416 computed
        assert table[1, :25].tolist() == table[0, :25].tolist()
        t.free(table[1, 25:(P + len(q) + ps - 1) // ps])


def test_fork_and_lock_in_pages():
    ps = 4
    t = RadixTree(32, page_size=ps)
    parent = np.arange(1, 11, dtype=np.int32)  # 2 full pages + 2 tokens
    table = np.full((4, 8), -1, np.int32)
    t.emit_rows([parent], table)
    pages = table[0, :2].copy()
    t.fork(parent, pages, [1, 2, 3], table)
    assert (table[1:4, :2] == pages).all() and (table[1:4, 2:] == -1).all()
    h, locked = t.lock([parent])
    assert locked.tolist() == [8] and t.stats()["locked_tokens"] == 2
    t.unlock(h)
    assert t.evict(100) == 2


def _expanded(table, ps):
    """One slot per position from rows of page ids (-1 pages stay -1)."""
    R, W = table.shape
    out = np.full((R, W * ps), -1, np.int64)
    for r in range(R):
        for j in range(W):
            if table[r, j] >= 0:
                out[r, j * ps:(j + 1) * ps] = table[r, j] * ps + np.arange(ps)
    return out


def _check_plan(plan, max_seq, rows, slots, group, cols=N.RC_DECODE_COLS):
    buf, info = plan.host, plan.info
    H, I = N.RC_PLAN_HEADER, N.RC_PLAN_ITEM
    items = buf[H:H + I * info.n_items].reshape(-1, I)
    mem = buf[H + I * info.n_items:H + I * info.n_items + info.n_members]
    cover = {m: [] for m in range(len(max_seq))}
    for rep, pb, pe, sp, mo, mc, _, _ in items:
        assert 1 <= mc <= max(1, cols // group) and pb < pe
        for m in mem[mo:mo + mc]:
            cover[int(m)].append((int(pb), int(pe)))
            assert np.array_equal(slots[rep, pb:pe], slots[rows[int(m)], pb:pe])
    for m, ranges in cover.items():
        ranges.sort()
        pos = 0
        for pb, pe in ranges:
            assert pb == pos
            pos = pe
        assert pos == max_seq[m]
    return items, mem


@pytest.mark.parametrize("ps", [2, 16])
def test_paged_decode_and_extend_plans(ps):
    g = np.random.default_rng(ps)
    doc = g.integers(0, 1000, 333).astype(np.int32)
    tails = [g.integers(0, 1000, n).astype(np.int32) for n in (5, 40, 17, 64, 1)]
    batch = [np.concatenate([doc, x]) for x in tails]
    t = RadixTree(4096, page_size=ps)
    table = np.full((len(batch) + 1, 256), -1, np.int32)
    t.emit_rows([doc], table, rows=[len(batch)])
    t.insert_rows([doc], table, [len(batch)])
    reserve = 3
    P, E = t.emit_rows(batch, table, reserve=reserve)
    assert (P == (333 // ps) * ps).all()  # the document's whole pages are shared, its partial page is not
    rows = np.arange(len(batch), dtype=np.int32)
    # cascade extend: every new token over its prefix and the new tokens before it
    plan = t.plan_extend(batch, P, E, group=4, chunk=128, rows=rows)
    seq = np.concatenate([p + np.arange(1, e + 1) for p, e in zip(P, E)])
    rows_of = np.repeat(rows, E)
    items, mem = _check_plan(plan, seq, rows_of, _expanded(table, ps), 4, cols=N.RC_EXTEND_SHARED_COLS)
    assert any(mc > 1 for *_, mc, _, _ in items)  # the shared pages are read for several tokens at once
    # decode after committing the batch
    t.insert_rows(batch, table, rows)
    lens = np.array([len(x) for x in batch], np.int32)
    plan = t.plan_decode(batch, lens + reserve, group=4, chunk=128, rows=rows)
    _check_plan(plan, lens + reserve, rows, _expanded(table, ps), 4)


def test_page_dictionary_holds_what_the_tree_holds():
    ps = 4
    A, B, C = [1, 2, 3, 4], [5, 6, 7, 8], [9, 9, 9, 9]
    t = RadixTree(32, page_size=ps)
    first = np.array(A + B + A + B + [3], np.int32)      # 4 full pages, 2 distinct contents
    second = np.array(C + A, np.int32)
    for seq in (first, second):
        ids = t.alloc(len(seq) // ps)
        t.insert(seq, ids)
    st_ = t.stats()
    assert st_["cached_tokens"] == 6 and st_["page_symbols"] == 3
    h, _ = t.lock([second])                               # the older sequence goes first anyway
    assert t.evict(1) == 4
    assert t.stats()["page_symbols"] == 2                 # B had no other holder; A is still in `second`
    m, _ = t.match(np.concatenate([first, [0]]).astype(np.int32))
    assert m == 0
    t.unlock(h)
    assert t.evict(100) == 2 and t.stats()["page_symbols"] == 0
    again = np.array(B + A + [0], np.int32)               # the numbers are reused after removal
    t.insert(again, t.alloc(2))
    assert t.stats()["page_symbols"] == 2
    m, got = t.match(np.concatenate([again, [7]]).astype(np.int32))
    assert m == 8 and len(got) == 2


def test_failed_paged_insert_leaves_no_symbols():
    t = RadixTree(8, page_size=2)
    seq = np.arange(1, 9, dtype=np.int32)                 # 4 pages
    with pytest.raises(RcError):
        t.insert(seq, np.array([0, 1, 2, 3], np.int32))    # never allocated: refused
    assert t.stats()["page_symbols"] == 0 and t.stats()["cached_tokens"] == 0
    t.insert(seq, t.alloc(4))
    assert t.stats()["page_symbols"] == 4


def test_large_batches_walk_on_several_threads_like_single_requests():
    # about a million tokens: the batch calls split their walks over host threads
    ps, g = 16, np.random.default_rng(11)
    stems = [g.integers(0, 50000, 2048 + 7 * i).astype(np.int32) for i in range(8)]
    t = RadixTree(1 << 16, page_size=ps)
    for x in stems:
        t.insert(x, t.alloc(len(x) // ps))
    batch = [np.concatenate([stems[i % 8][:g.integers(1000, len(stems[i % 8]) + 1)],
                             g.integers(0, 50000, g.integers(1, 2200)).astype(np.int32)]) for i in range(512)]
    assert sum(map(len, batch)) > 1 << 20
    want = []
    for x in batch:
        m, ids = t.match(x)
        want.append((m, ids))
    table = np.full((len(batch), 512), -1, np.int32)
    P, E = t.emit_rows(batch, table, reserve=3)
    for b, (m, ids) in enumerate(want):
        assert P[b] == m and (table[b, :m // ps] == ids).all()
    h, locked = t.lock(batch)
    assert locked.tolist() == [m for m, _ in want]
    t.unlock(h)
    rows = np.arange(len(batch), dtype=np.int32)
    plan = t.plan_decode(batch, P.astype(np.int32) + 1, group=4, chunk=4096, rows=rows,
                         lengths=P.astype(np.int64))
    _check_plan(plan, P + 1, rows, _expanded(table, ps), 4)


@pytest.mark.parametrize("ps", [0, -4, 3, 12, 2048])
def test_paged_tree_rejects_bad_page_sizes(ps):
    with pytest.raises((RcError, ValueError)):
        RadixTree(64, page_size=ps)


def test_paged_calls_reject_mismatched_page_rows():
    t = RadixTree(16, page_size=4)
    seq = np.arange(1, 10, dtype=np.int32)          # 2 full pages + 1 token
    with pytest.raises((RcError, ValueError)):
        t.insert(seq, t.alloc(3))                   # one page id per full page: 2, not 3
    assert t.stats()["cached_tokens"] == 0 and t.stats()["page_symbols"] == 0
    table = np.full((1, 2), -1, np.int32)           # 9 tokens + 0 reserve need 3 pages
    with pytest.raises(RcError) as e:
        t.emit_rows([seq], table)
    assert e.value.status == N.RC_ERR_RANGE


def test_full_match_flag_in_pages():
    # RC_EMIT_FULL_MATCH reuses every whole cached page: the model's match of a
    # probe one token longer; the partial last page is new
    ps = 4
    t, ref = RadixTree(32, page_size=ps), PagedRadixRef(32, ps)
    seq = list(range(100, 110))  # 2 whole pages + 2 tokens
    table = np.full((2, 8), -1, np.int32)
    rows, P, E = ref.emit_rows([seq])
    t.emit_rows([seq], table)
    ref.insert(seq, rows[0])
    t.insert_rows([seq], table, np.zeros(1, np.int32))
    t.free(table[0, 2:3])
    ref.free_pages(rows[0][2:3])
    m, ids = ref.match(seq + [-1])
    new = np.zeros(len(seq), np.int32)
    entries = np.zeros(1, np.int64)
    Pn, En = t.emit_rows([seq], table, rows=[1], full_match=True, row_entries=entries, new_slots=new)
    assert (int(Pn[0]), int(En[0])) == (m, len(seq) - m) == (8, 2)
    assert table[1, :2].tolist() == ids and entries[0] == 3
    assert new[:2].tolist() == [table[1, 2] * ps + 0, table[1, 2] * ps + 1]
