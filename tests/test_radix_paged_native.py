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
            Pn, En = tree.emit_rows(batch, table, reserve=reserve)
            assert Pn.tolist() == P and En.tolist() == E
            for b, r in enumerate(rows):
                assert table[b, :len(r)].tolist() == r
            if commit:
                for b, t in enumerate(batch):
                    canon, _ = ref.insert(t, rows[b])
                    rows[b][:len(canon)] = canon
                tree.insert_rows(batch, table, np.arange(len(batch), dtype=np.int32))
                for b, r in enumerate(rows):
                    assert table[b, :len(r)].tolist() == r
            running.append((batch, rows, commit, P))
        elif op[0] == "release" and running:
            batch, rows, commit, P = running.pop(op[1] % len(running))
            own = []
            for t, r, p in zip(batch, rows, P):
                own += r[(len(t) // ps if commit else p // ps):]  # pages the tree does not hold
            ref.free_pages(own)
            tree.free(np.array(own, np.int32))
        elif op[0] == "match":
            m, ids = tree.match(op[1])
            assert (m, ids.tolist()) == ref.match(op[1])
        assert tree.stats()["free_slots"] == len(ref.free)
    n = len(ref.free)
    assert tree.alloc(n).tolist() == ref.alloc(n)


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


def _check_plan(plan, max_seq, rows, slots, group):
    buf, info = plan.host, plan.info
    H, I = N.RC_PLAN_HEADER, N.RC_PLAN_ITEM
    items = buf[H:H + I * info.n_items].reshape(-1, I)
    mem = buf[H + I * info.n_items:H + I * info.n_items + info.n_members]
    cover = {m: [] for m in range(len(max_seq))}
    for rep, pb, pe, sp, mo, mc, _, _ in items:
        assert 1 <= mc <= max(1, 128 // group) and pb < pe
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
    items, mem = _check_plan(plan, seq, rows_of, _expanded(table, ps), 4)
    assert any(mc > 1 for *_, mc, _, _ in items)  # the shared pages are read for several tokens at once
    # decode after committing the batch
    t.insert_rows(batch, table, rows)
    lens = np.array([len(x) for x in batch], np.int32)
    plan = t.plan_decode(batch, lens + reserve, group=4, chunk=128, rows=rows)
    _check_plan(plan, lens + reserve, rows, _expanded(table, ps), 4)
