"""Decode and cascade-extend plans from the native tree (host only).

Every plan is checked against what its definition requires, with a table
built by the tree itself:
  * each member's items cover its positions [0, max_seq) exactly once, with
    distinct split indices below its split count;
  * an item's positions hold the same slots in every member's table row as
    in the representative row the kernel reads them through;
  * members per item stay within max(1, cols / group), cols = 128 columns for
    decode plans and 256 for cascade extend plans;
  * items flagged as a request's own positions (the only items the decode
    kernel lets store the current token) have one member and cover a suffix
    of its positions, every position past its committed tokens included,
    never a range that another request reads.
"""
import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from prefix_shared_kv_amd import RadixTree
from prefix_shared_kv_amd import _native as N


def parse(plan):
    buf, info = plan.host, plan.info
    H, I = N.RC_PLAN_HEADER, N.RC_PLAN_ITEM
    items = buf[H:H + I * info.n_items].reshape(-1, I)
    mem = buf[H + I * info.n_items:H + I * info.n_items + info.n_members]
    nsplit = buf[H + I * info.n_items + info.n_members:]
    return items, mem, nsplit


def check_plan(plan, max_seq, rows, table, group, own_from=None, cols=N.RC_DECODE_COLS):
    items, mem, nsplit = parse(plan)
    max_m = max(1, cols // group)
    assert plan.info.max_cols == max_m * group
    cover = {m: [] for m in range(len(max_seq))}
    own = {m: [] for m in range(len(max_seq))}
    for rep, pb, pe, sp, mo, mc, flags, _ in items:
        assert 1 <= mc <= max_m and pb < pe
        assert flags & ~N.RC_PLAN_ITEM_OWN == 0
        if flags & N.RC_PLAN_ITEM_OWN:
            assert mc == 1
            own[int(mem[mo])].append((int(pb), int(pe)))
        for m in mem[mo:mo + mc]:
            m = int(m)
            cover[m].append((int(pb), int(pe), int(sp)))
            # the kernel reads the range through rep's row for every member
            assert np.array_equal(table[rep, pb:pe], table[rows[m], pb:pe]), (m, pb, pe)
    for m, rs in own.items():
        if not rs:
            assert own_from is None or own_from[m] >= max_seq[m]
            continue
        rs.sort()
        assert rs[-1][1] == max_seq[m], (m, rs)  # a suffix of the member's positions ...
        assert all(a[1] == b[0] for a, b in zip(rs, rs[1:])), (m, rs)
        assert all(pe <= rs[0][0] for pb, pe, _ in cover[m] if (pb, pe) not in rs), (m, rs)
        if own_from is not None:  # ... holding every position past its committed tokens
            assert rs[0][0] <= own_from[m], (m, rs, own_from[m])
            # members are requests: no other request reads a slot of these positions
            others = np.concatenate([table[rows[x], :max_seq[x]] for x in own if x != m] or [np.zeros(0, np.int32)])
            mine = np.concatenate([table[rows[m], pb:pe] for pb, pe in rs])
            assert not np.isin(mine, others).any(), (m, rs)
    for m, ranges in cover.items():
        ranges.sort()
        pos = 0
        for pb, pe, _ in ranges:
            assert pb == pos, (m, ranges)
            pos = pe
        assert pos == max_seq[m], (m, ranges, max_seq[m])
        splits = sorted(sp for _, _, sp in ranges)
        assert len(set(splits)) == len(splits) and splits[-1] < nsplit[m] <= plan.info.max_splits
    return items, mem


def build(seqs, pool=20000, insert=None):
    """A tree holding `insert` (default: all of seqs) with table rows for seqs."""
    t = RadixTree(pool)
    for s in (seqs if insert is None else insert):
        m, pre = t.match(np.concatenate([s, [-1]]).astype(np.int32))
        t.insert(s, np.concatenate([pre, t.alloc(len(s) - m)]).astype(np.int32))
    return t


def test_extend_plan_reads_a_shared_document_once_per_token_group():
    g = np.random.default_rng(1)
    doc = g.integers(0, 1000, 300).astype(np.int32)
    labels = [g.integers(1000, 2000, n).astype(np.int32) for n in (2, 5, 16, 1, 9)]
    for i, lab in enumerate(labels):  # distinct first tokens: no sharing among the labels
        lab[0] = 5000 + i
    t = build([doc])
    batch = [np.concatenate([doc, lab]) for lab in labels]
    table = np.full((len(batch), 400), -1, np.int32)
    P, E = t.emit_rows(batch, table)
    assert P.tolist() == [300] * 5 and E.tolist() == [2, 5, 16, 1, 9]
    group = 8
    plan = t.plan_extend(batch, P, E, group)
    rows = np.repeat(np.arange(5), E)
    max_seq = np.concatenate([p + np.arange(1, e + 1) for p, e in zip(P, E)])
    items, mem = check_plan(plan, max_seq, rows, table, group, cols=N.RC_EXTEND_SHARED_COLS)
    doc_items = [it for it in items if it[1] == 0 and it[2] == 300]
    # 33 new tokens in groups of 256 / 8 = 32: the document is read by 2 items, not 5 or 33
    assert sorted(int(it[5]) for it in doc_items) == [1, 32]
    own = [it for it in items if it[1] >= 300]
    assert len(own) == 33 and all(it[5] == 1 for it in own)
    assert plan.info.batch == 33 and plan.info.max_splits == 2


def test_extend_plan_without_a_cached_prefix():
    t = RadixTree(1000)
    batch = [np.arange(10, 30, dtype=np.int32), np.arange(50, 57, dtype=np.int32)]
    table = np.full((2, 32), -1, np.int32)
    P, E = t.emit_rows(batch, table)
    assert P.tolist() == [0, 0]
    plan = t.plan_extend(batch, P, E, 4)
    check_plan(plan, np.concatenate([np.arange(1, 21), np.arange(1, 8)]), np.repeat([0, 1], E), table, 4,
               cols=N.RC_EXTEND_SHARED_COLS)
    assert plan.info.shared_items == 0


def test_extend_plan_rejects_lengths_past_the_tokens():
    t = RadixTree(100)
    with pytest.raises(N.RcError):
        t.plan_extend([np.arange(5, dtype=np.int32)], [3], [3], 4)


@st.composite
def tree_batches(draw):
    vocab = draw(st.integers(2, 5))
    n_seq = draw(st.integers(1, 6))
    base = draw(st.lists(st.integers(0, vocab - 1), min_size=1, max_size=60))
    seqs = []
    for _ in range(n_seq):
        cut = draw(st.integers(0, len(base)))
        tail = draw(st.lists(st.integers(0, vocab - 1), min_size=1, max_size=30))
        seqs.append(np.array(base[:cut] + tail, np.int32))
    n_cached = draw(st.integers(0, n_seq))
    n_new = [draw(st.integers(1, 12)) for _ in range(n_seq)]
    group = draw(st.sampled_from([1, 4, 8, 32]))
    chunk = draw(st.sampled_from([3, 16, 64, 4096]))
    return seqs, n_cached, n_new, group, chunk


@settings(max_examples=120, deadline=None)
@given(tree_batches())
def test_plans_cover_every_context_with_shared_slots(case):
    seqs, n_cached, n_new, group, chunk = case
    t = build(seqs, insert=seqs[:n_cached])
    g = np.random.default_rng(len(seqs) + n_cached)
    batch = [np.concatenate([s, 100 + g.integers(0, 3, k)]).astype(np.int32) for s, k in zip(seqs, n_new)]
    reserve = 4
    table = np.full((len(batch), max(len(b) for b in batch) + reserve), -1, np.int32)
    P, E = t.emit_rows(batch, table, reserve=reserve)
    # cascade extend over the new tokens
    plan = t.plan_extend(batch, P, E, group, chunk)
    rows = np.repeat(np.arange(len(batch)), E)
    max_seq = np.concatenate([p + np.arange(1, e + 1) for p, e in zip(P, E)])
    check_plan(plan, max_seq, rows, table, group, cols=N.RC_EXTEND_SHARED_COLS)
    # token i of request b attends over positions [0, P_b + i]
    assert plan.seq_lens.tolist() == max_seq.tolist()
    # decode plan after commit: contexts up to the reserved slots
    t.insert_rows(batch, table, np.arange(len(batch), dtype=np.int32))
    lens = np.array([len(b) for b in batch])
    plan = t.plan_decode(batch, lens + reserve, group, chunk)
    check_plan(plan, lens + reserve, np.arange(len(batch)), table, group, own_from=lens)
    # the shared (cached) part of a context is never flagged as a request's own
    for rep, pb, pe, sp, mo, mc, flags, _ in plan.items():
        if mc > 1:
            assert flags == 0


def test_launch_order_puts_the_longer_running_class_first():
    # a long shared prefix and short own tails: wide items first; short shared
    # heads and long own tails: narrow items first (a narrow item's length counts
    # double: one wave streams it against a wide item's four)
    g = np.random.default_rng(3)
    for shared, own, want in ((2048, 64, 0), (256, 2000, 1), (1000, 600, 1), (1000, 400, 0)):
        stem = g.integers(0, 1000, shared).astype(np.int32)
        batch = [np.concatenate([stem, g.integers(0, 1000, own).astype(np.int32)]) for _ in range(64)]
        t = RadixTree(1 << 20)
        table = np.full((64, shared + own + 8), -1, np.int32)
        t.emit_rows(batch, table)
        t.insert_rows(batch, table, np.arange(64, dtype=np.int32))
        lens = np.array([len(x) for x in batch], np.int32)
        plan = t.plan_decode(batch, lens, group=4, chunk=4096)
        items = plan.items()
        nb = plan.info.narrow_begin
        lw = int((items[:nb, 2] - items[:nb, 1]).max())
        ln = int((items[nb:, 2] - items[nb:, 1]).max())
        assert (lw, ln) == (shared, own) and plan.info.narrow_first == want, (shared, own)


def test_unshared_and_cascade_plans_choose_their_launch_order():
    # an unshared plan has only narrow items (one member each): they go first;
    # a cascade plan over a long document with short label branches keeps its
    # wide document ranges first
    from prefix_shared_kv_amd import api
    plan = api.plan_decode_unshared(np.array([5000, 300, 1], np.int32), 4, 4096)
    assert plan.info.narrow_begin == 0 and plan.info.narrow_first == 1
    g = np.random.default_rng(5)
    doc = g.integers(0, 1000, 4096).astype(np.int32)
    batch = [np.concatenate([doc, g.integers(0, 1000, n).astype(np.int32)]) for n in (2, 9, 16, 5) * 16]
    t = RadixTree(1 << 20)
    table = np.full((len(batch), 4200), -1, np.int32)
    t.emit_rows([doc], table[:1])
    t.insert_rows([doc], table[:1], np.zeros(1, np.int32))
    P, E = t.emit_rows(batch, table)
    plan = t.plan_extend(batch, P, E, group=8, chunk=1024)
    assert plan.info.narrow_begin > 0 and plan.info.narrow_first == 0


def test_items_run_longest_first_within_each_class():
    # without bins: wide items by members x positions, narrow items by
    # positions alone (one wave streams a narrow range whatever its members)
    g = np.random.default_rng(21)
    stems = [g.integers(0, 1000, n).astype(np.int32) for n in (700, 300)]
    batch = []
    for k, stem in enumerate(stems):
        for i in range(4 if k else 6):  # 6 and 4 members: wide with group 4 past 4 members
            batch.append(np.concatenate([stem, g.integers(2000, 3000, int(g.integers(50, 900))).astype(np.int32)]))
    t = RadixTree(1 << 20)
    table = np.full((len(batch), 2000), -1, np.int32)
    t.emit_rows(batch, table)
    t.insert_rows(batch, table, np.arange(len(batch), dtype=np.int32))
    lens = np.array([len(x) for x in batch], np.int32)
    plan = t.plan_decode(batch, lens, group=4, chunk=4096)
    items, _ = check_plan(plan, lens, np.arange(len(batch)), table, 4, own_from=lens)
    nb = plan.info.narrow_begin
    wide_cost = (items[:nb, 2] - items[:nb, 1]) * items[:nb, 5]
    narrow_len = items[nb:, 2] - items[nb:, 1]
    assert nb >= 1 and np.all(np.diff(wide_cost) <= 0) and np.all(np.diff(narrow_len) <= 0)
    # the 4-member stem is narrow (16 columns) and sorts among the own ranges by its length
    assert any(it[5] == 4 for it in items[nb:])
