"""The C++ radix tree and slot allocator against the brute-force model in
oracle/radix_ref.py: matched lengths, slot lists, table rows and the free
list must agree exactly on random operation sequences.  Tree shapes may
differ; only observable outputs are compared."""
import ctypes as C

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle.radix_ref import OutOfSlots, RadixRef
from prefix_shared_kv_amd import RadixTree, RcError
from prefix_shared_kv_amd import _native as N
from prefix_shared_kv_amd import api


def _seq(draw, base, vocab):
    # sequences built from a few shared stems so prefixes collide often
    stem = draw(st.sampled_from(base))
    tail = draw(st.lists(st.integers(0, vocab - 1), min_size=0, max_size=6))
    cut = draw(st.integers(0, len(stem)))
    return stem[:cut] + tail


@st.composite
def scenarios(draw):
    vocab = draw(st.sampled_from([3, 5, 50]))
    base = [draw(st.lists(st.integers(0, vocab - 1), min_size=1, max_size=10)) for _ in range(3)]
    ops = []
    for _ in range(draw(st.integers(1, 25))):
        kind = draw(st.sampled_from(["match", "emit_insert", "emit_insert", "alloc_free"]))
        if kind == "emit_insert":
            batch = [_seq(draw, base, vocab) or [0] for _ in range(draw(st.integers(1, 3)))]
            reserve = draw(st.integers(0, 2))
            ops.append((kind, batch, reserve))
        elif kind == "match":
            ops.append((kind, _seq(draw, base, vocab)))
        else:
            ops.append((kind, draw(st.integers(0, 4))))
    perm = draw(st.booleans())
    return ops, perm


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(scenarios())
def test_tree_matches_bruteforce(sc):
    ops, perm = sc
    S = 120
    order = np.random.default_rng(len(ops)).permutation(S).astype(np.int32) if perm else None
    tree, ref = RadixTree(S, order), RadixRef(S, order)
    table = np.full((4, 64), -1, np.int32)
    for op in ops:
        if op[0] == "match":
            got = tree.match(op[1])
            want = ref.match(op[1])
            assert got[0] == want[0]
            assert got[1].tolist() == want[1]
        elif op[0] == "alloc_free":
            n = op[1]
            try:
                want = ref.alloc(n)
            except OutOfSlots:
                with pytest.raises(RcError):
                    tree.alloc(n)
                continue
            got = tree.alloc(n)
            assert got.tolist() == want
            tree.free(got)
            ref.free_slots(want)
        else:
            _, batch, reserve = op
            try:
                rows_w, P_w, E_w = ref.emit_rows(batch, reserve)
            except OutOfSlots:
                before = tree.stats()["free_slots"]
                with pytest.raises(RcError) as ei:
                    tree.emit_rows(batch, table, reserve=reserve)
                assert ei.value.status == N.RC_ERR_NOMEM
                assert tree.stats()["free_slots"] == before
                continue
            entries = np.zeros(len(batch), np.int64)
            new_slots = np.full(sum(len(x) for x in batch) + 1, -7, np.int32)
            P, E = tree.emit_rows(batch, table, reserve=reserve, row_entries=entries, new_slots=new_slots)
            assert P.tolist() == P_w and E.tolist() == E_w
            o = 0
            for b, toks in enumerate(batch):
                n = len(toks) + reserve
                assert table[b, :n].tolist() == rows_w[b]
                assert entries[b] == n
                # the new tokens' slots: positions P_b .. n_b - 1 of the model's row
                assert new_slots[o:o + E_w[b]].tolist() == rows_w[b][P_w[b]:P_w[b] + E_w[b]]
                o += E_w[b]
            assert (new_slots[o:] == -7).all()
            # commit each request's prompt; rows get the tree's slots back
            if len(ops) % 2:
                for b, toks in enumerate(batch):
                    canon, n_new = tree.insert(toks, table[b, :len(toks)])
                    canon_w, n_new_w = ref.insert(toks, rows_w[b][:len(toks)])
                    assert canon.tolist() == canon_w and n_new == n_new_w
            else:  # the batched commit
                before = table.copy()
                changed = tree.insert_rows(batch, table, list(range(len(batch))))
                for b, toks in enumerate(batch):
                    canon_w, _ = ref.insert(toks, rows_w[b][:len(toks)])
                    assert table[b, :len(toks)].tolist() == canon_w
                    assert bool(changed[b]) == (before[b, :len(toks)].tolist() != canon_w)
                # reserved decode slots are not used here: give them back
            # the reserved decode slots go back (free_rows from each prompt's end to its row's end)
            tree.free_rows(np.arange(len(batch)), table, [len(x) for x in batch], entries)
            for b, toks in enumerate(batch):
                if reserve:
                    ref.free_slots(rows_w[b][len(toks):len(toks) + reserve])
        assert tree.stats()["free_slots"] == ref.num_free()
    assert list(ref.free)[:5] == tree.alloc(min(5, ref.num_free())).tolist()


def test_split_and_stats():
    t = RadixTree(64)
    a = t.alloc(6)
    t.insert([1, 2, 3, 4, 5, 6], a)
    b = t.alloc(3)
    canon, n_new = t.insert([1, 2, 3, 9, 9, 9], np.concatenate([a[:3], b]))
    assert n_new == 3 and canon.tolist() == a[:3].tolist() + b.tolist()
    s = t.stats()
    assert s["splits"] == 1 and s["nodes"] == 3 and s["cached_tokens"] == 9
    m, sl = t.match([1, 2, 3, 9, 9, 9, 7])
    assert m == 6 and sl.tolist() == canon.tolist()


def test_insert_rejects_bad_slots_atomically():
    t = RadixTree(16)
    a = t.alloc(3)
    t.insert([1, 2, 3], a)
    free_before = t.stats()["free_slots"]
    with pytest.raises(RcError):
        t.insert([1, 2, 3, 4], [a[0], a[1], a[2], 15])  # slot 15 is still free
    with pytest.raises(RcError):
        t.insert([5, 6], [a[0], a[1]])  # slots already held by the tree
    with pytest.raises(RcError):
        t.free([a[0]])  # held by the tree
    assert t.stats()["free_slots"] == free_before
    assert t.match([1, 2, 3, 4])[0] == 3


def test_free_order_must_be_a_permutation():
    with pytest.raises(RcError):
        RadixTree(4, np.array([0, 1, 1, 3], np.int32))


def test_fork_shares_the_prefix_rows():
    t = RadixTree(32)
    table = np.full((4, 16), -1, np.int32)
    parent = t.alloc(5)
    t.fork([7, 7, 8, 9, 1], parent, [1, 2, 3], table)
    for r in (1, 2, 3):
        assert table[r, :5].tolist() == parent.tolist()
    # a child extending the forked prefix matches all of it
    P, E = t.emit_rows([[7, 7, 8, 9, 1, 4, 4]], table, rows=[1])
    assert P.tolist() == [5] and E.tolist() == [2]


def test_gpt2_bookkeeping_through_the_native_tree():
    t = RadixTree(1024)
    prefix = list(range(100, 509))
    table = np.full((3, 512), -1, np.int32)
    P, E = t.emit_rows([prefix], table)
    assert (P[0], E[0]) == (0, 409)
    t.insert(prefix, table[0, :409])
    P, E = t.emit_rows([prefix + list(range(9000, 9008)), prefix + list(range(9100, 9107))], table, rows=[1, 2])
    assert [(int(p), int(e), int(p + e)) for p, e in zip(P, E)] == [(409, 8, 417), (409, 7, 416)]


def test_token_batch_lengths_equal_sliced_lists():
    # a prefix of each request given by tok_len walks exactly like the sliced token lists
    g = np.random.default_rng(3)
    t = RadixTree(4000)
    base = g.integers(0, 50, 300).astype(np.int32)
    seqs = [np.concatenate([base[:g.integers(50, 300)], g.integers(0, 50, g.integers(1, 40))]).astype(np.int32)
            for _ in range(12)]
    for s in seqs[:6]:
        m, pre = t.match(np.concatenate([s, [-1]]))
        t.insert(s, np.concatenate([pre, t.alloc(len(s) - m)]))
    tb = api.TokenBatch(seqs)
    lengths = [int(g.integers(0, len(s) + 1)) for s in seqs]
    max_seq = [len(s) + 3 for s in seqs]
    a = t.plan_decode([s[:n] for s, n in zip(seqs, lengths)], max_seq, 4, 64)
    b = t.plan_decode(tb, max_seq, 4, 64, lengths=lengths)
    assert np.array_equal(a.host, b.host)
    with pytest.raises(RcError):
        t.plan_decode(tb, max_seq, 4, 64, lengths=[len(seqs[0]) + 1] + lengths[1:])
    with pytest.raises(RcError):
        t.insert_rows(tb, np.zeros((12, 400), np.int32), list(range(12)), lengths=[-1] + lengths[1:])


@pytest.mark.parametrize("ps", [1, 4])
def test_first_changed_marks_where_each_row_starts_to_differ(ps):
    # rows reused by batch after batch: first_changed[b] is the first entry of
    # row rows[b] that the call changed (its entry count if none), and no entry
    # before it changed; later batches share prefixes with the rows' earlier
    # contents, so the changes start anywhere from 0 to past the prefix
    g = np.random.default_rng(ps)
    stems = [g.integers(0, 40, g.integers(4, 60)).astype(np.int32) for _ in range(5)]
    t = RadixTree(1 << 16, page_size=ps) if ps > 1 else RadixTree(1 << 16)
    table = np.full((6, 80), -1, np.int32)
    seen = set()
    for it in range(60):
        B = int(g.integers(1, 5))
        rows = g.permutation(6)[:B].astype(np.int32)
        batch = [np.concatenate([stems[g.integers(0, 5)][:g.integers(0, 60)],
                                 g.integers(0, 40, g.integers(1, 8)).astype(np.int32)]) for _ in range(B)]
        reserve = int(g.integers(0, 3))
        before = table.copy()
        first = np.zeros(B, np.int64)
        t.emit_rows(batch, table, rows=rows, reserve=reserve, first_changed=first)
        for b, r in enumerate(rows):
            n = -(-(len(batch[b]) + reserve) // ps)
            diff = np.flatnonzero(table[r, :n] != before[r, :n])
            assert first[b] == (diff[0] if len(diff) else n), (it, b)
            assert (table[r, n:] == before[r, n:]).all()
            seen.add(min(int(first[b]), 3))
        if it % 2 == 0:
            t.insert_rows(batch, table, rows)
    assert {0, 3} <= seen  # rows changed from their first entry, and from later ones


def test_full_match_flag_stores_a_fully_cached_sequence_without_new_tokens():
    # the usual match keeps at least one token to run; with RC_EMIT_FULL_MATCH a
    # sequence already cached gets no new tokens (storing K/V computed elsewhere)
    t, ref = RadixTree(64), RadixRef(64)
    seq = [5, 6, 7, 8, 9]
    table = np.full((2, 16), -1, np.int32)
    P, E = t.emit_rows([seq], table)
    rows_w, P_w, E_w = ref.emit_rows([seq], 0)
    assert (P.tolist(), E.tolist()) == (P_w, E_w) == ([0], [5])
    t.insert(seq, table[0, :5])
    ref.insert(seq, rows_w[0])
    P, E = t.emit_rows([seq], table, rows=[1])
    assert (P.tolist(), E.tolist()) == ([4], [1])  # capped at n - 1
    t.free(table[1, 4:5])
    new = np.zeros(6, np.int32)
    P, E = t.emit_rows([seq], table, rows=[1], full_match=True, new_slots=new)
    m, slots = ref.match(seq + [-1])  # the model's uncapped match: a probe one token longer
    assert (P.tolist(), E.tolist()) == ([m], [0]) and table[1, :5].tolist() == slots
    with pytest.raises(RcError) as e:  # unknown flag bits
        N.check(N.lib.rc_radix_emit_rows(t._h, 0, None, np.zeros(1, np.int64).ctypes.data_as(C.c_void_p), 0, None,
                                         None, 0, 16, None, None, 4, None, None, None, None))
    assert e.value.status == N.RC_ERR_ARG


@pytest.mark.parametrize("ps", [1, 4, 16])
def test_decode_steps_follow_the_table_rows(ps):
    # step t of request b: the token at position base_b + t, its slot read from the row
    # (row[p], or row[p // ps] * ps + p % ps for pages) and its context p + 1 positions
    from prefix_shared_kv_amd import api
    g = np.random.default_rng(ps)
    rows = np.array([2, 0, 3], np.int32)
    base = np.array([0, 17, 40], np.int32)
    T = 9
    entries = np.array([-(-(int(x) + T) // ps) for x in base], np.int64)
    table = np.full((4, 64), -1, np.int32)
    for r, e in zip(rows, entries):
        table[r, :e] = g.permutation(1000)[:e]
    slots, seq = api.decode_steps(table, rows, base, T, ps, row_entries=entries)
    for t in range(T):
        for b in range(3):
            p = int(base[b]) + t
            assert slots[t, b] == table[rows[b], p // ps] * ps + p % ps
            assert seq[t, b] == p + 1
    with pytest.raises(RcError):  # one step past the first request's reserved entries
        api.decode_steps(table, rows, base, int(entries[0]) * ps + 1, ps, row_entries=entries)
    short = table.copy()
    short[rows[2], entries[2] - 1] = -1
    with pytest.raises(RcError):  # a position whose entry holds no slot
        api.decode_steps(short, rows, base, T, ps, row_entries=entries)
    with pytest.raises(RcError):
        api.decode_steps(table, rows, base, T, 3)
