"""GPU parity for a paged KV pool (page_size > 1): req_to_token holds page ids,
one per page_size positions, pages drawn in shuffled order.  Every output must
equal, bit for bit, the same call with the table expanded to one slot per
position (page * page_size + offset: the same slots, so the same arithmetic),
and the oracle within max-abs 2e-2 (bf16) / 1e-4 (fp32).  Page ids outside the
pool are flagged and never dereferenced."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from prefix_shared_kv_amd import KVShape, api
from synth import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DT = {"f32": torch.float32, "bf16": torch.bfloat16}
HEADS = {"bf16": (32, 8, 128), "f32": (8, 2, 64)}


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def dev(a, gpu):
    return torch.from_numpy(np.ascontiguousarray(a)).to(gpu)


def tables(g, lens, ps, n_pages, rows):
    """Page table [R, max pages] and the equivalent per-position slot table [R, max pages * ps]."""
    need = [(n + ps - 1) // ps for n in lens]
    order = g.permutation(n_pages).astype(np.int32)
    mp = max(need) + 1
    pt = np.full((len(rows) + 2, mp), -1, np.int32)
    st = np.full((len(rows) + 2, mp * ps), -1, np.int32)
    used = 0
    for b, k in enumerate(need):
        pg = order[used:used + k]
        used += k
        pt[rows[b], :k] = pg
        st[rows[b], :k * ps] = (pg[:, None] * ps + np.arange(ps)[None, :]).reshape(-1)
    return pt, st


def fill_pool(g, S, Hkv, D, dtype):
    x = g.standard_normal((S, Hkv, D)).astype(np.float32)
    return W.round_bf16(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ps", [4, 16, 64, 256, 1024])
def test_paged_extend_equals_expanded_table(gpu, dtype, ps):
    g = np.random.default_rng(ps)
    Hq, Hkv, D = HEADS[dtype]
    P_list = [0, 1, 63, 64, 130, 300, 5]
    E_list = [70, 1, 65, 0, 33, 129, 8]
    B = len(P_list)
    rows = (np.arange(B) + 1).astype(np.int32)
    n_pages = sum((p + ps - 1) // ps for p in P_list) + 8
    S = n_pages * ps
    pool = fill_pool(g, S, Hkv, D, dtype), fill_pool(g, S, Hkv, D, dtype)
    pt, st = tables(g, P_list, ps, n_pages, rows)
    T = sum(E_list)
    rnd = lambda *s: (W.round_bf16 if dtype == "bf16" else (lambda x: x))(g.standard_normal(s).astype(np.float32))
    q, kn, vn = rnd(T, Hq, D), rnd(T, Hkv, D), rnd(T, Hkv, D)
    start = np.concatenate([[0], np.cumsum(E_list)[:-1]]).astype(np.int32)
    to = lambda a: torch.from_numpy(a).to(gpu).to(DT[dtype])
    kp, vp = to(pool[0]), to(pool[1])
    outs = []
    for shape, tab in ((KVShape(Hq, Hkv, D, DT[dtype], S, ps), pt), (KVShape(Hq, Hkv, D, DT[dtype], S), st)):
        o = torch.full((T, Hq, D), 7.0, device=gpu, dtype=DT[dtype])
        err = torch.zeros(1, dtype=torch.int32, device=gpu)
        api.set_error_word(err)
        try:
            api.extend_attention(shape, o, to(q), to(kn), to(vn), kp, vp, dev(tab, gpu), dev(np.array(P_list, np.int32), gpu),
                                 dev(np.array(E_list, np.int32), gpu), dev(start, gpu), max(E_list), 1.0 / np.sqrt(D),
                                 rows=dev(rows, gpu))
            torch.cuda.synchronize()
        finally:
            api.set_error_word(None)
        assert int(err.item()) == 0
        outs.append(o)
    assert torch.equal(outs[0], outs[1]), "paged table and expanded table give different bits"
    got = host(outs[0])
    for b in range(B):
        E, P = E_list[b], P_list[b]
        if E == 0:
            continue
        s0 = start[b]
        slots = st[rows[b], :P]
        K = np.concatenate([pool[0][slots], kn[s0:s0 + E]])
        V = np.concatenate([pool[1][slots], vn[s0:s0 + E]])
        want = A.extend(q[s0:s0 + E], K, V, P, 1.0 / np.sqrt(D))
        e = float(np.max(np.abs(got[s0:s0 + E] - want)))
        assert e <= TOL[dtype], f"request {b}: max abs error {e:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ps", [4, 16, 64, 256, 1024])
def test_paged_decode_with_store_equals_expanded_table(gpu, dtype, ps):
    g = np.random.default_rng(100 + ps)
    Hq, Hkv, D = HEADS[dtype]
    L = [1, 5, 64, 65, 130, 700, 2049, 33]  # context lengths, the current token included
    B = len(L)
    rows = (np.arange(B) + 1).astype(np.int32)
    n_pages = sum((n + ps - 1) // ps for n in L) + 4
    S = n_pages * ps
    base = fill_pool(g, S, Hkv, D, dtype), fill_pool(g, S, Hkv, D, dtype)
    pt, st = tables(g, L, ps, n_pages, rows)
    rnd = lambda *s: (W.round_bf16 if dtype == "bf16" else (lambda x: x))(g.standard_normal(s).astype(np.float32))
    q, kn, vn = rnd(B, Hq, D), rnd(B, Hkv, D), rnd(B, Hkv, D)
    new_slots = np.array([st[rows[b], L[b] - 1] for b in range(B)], np.int32)
    to = lambda a: torch.from_numpy(a).to(gpu).to(DT[dtype])
    plan = api.plan_decode_unshared(L, Hq // Hkv, 256, rows=rows)
    plan.to(gpu)
    results = []
    for shape, tab in ((KVShape(Hq, Hkv, D, DT[dtype], S, ps), pt), (KVShape(Hq, Hkv, D, DT[dtype], S), st)):
        kp, vp = to(base[0]), to(base[1])
        o = torch.empty(B, Hq, D, device=gpu, dtype=DT[dtype])
        ws = torch.empty(api.decode_workspace_bytes(shape, plan), dtype=torch.uint8, device=gpu)
        err = torch.zeros(1, dtype=torch.int32, device=gpu)
        api.set_error_word(err)
        try:
            api.decode_attention(shape, o, to(q), kp, vp, dev(tab, gpu), dev(np.array(L, np.int32), gpu), plan,
                                 1.0 / np.sqrt(D), ws, k_new=to(kn), v_new=to(vn), new_slots=dev(new_slots, gpu))
            torch.cuda.synchronize()
        finally:
            api.set_error_word(None)
        assert int(err.item()) == 0
        results.append((o, kp, vp))
    assert torch.equal(results[0][0], results[1][0]), "paged and expanded decode outputs differ"
    assert torch.equal(results[0][1], results[1][1]) and torch.equal(results[0][2], results[1][2])
    got = host(results[0][0])
    pk, pv = base[0].copy(), base[1].copy()
    pk[new_slots], pv[new_slots] = kn, vn
    for b in range(B):
        slots = st[rows[b], :L[b]]
        want = A.decode(q[b], pk[slots], pv[slots], 1.0 / np.sqrt(D))
        e = float(np.max(np.abs(got[b] - want)))
        assert e <= TOL[dtype], f"request {b} (L={L[b]}): max abs error {e:.3e}"


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 8, 2, 128), ("bf16", 32, 1, 128), ("bf16", 16, 4, 64),
                                             ("f32", 8, 2, 64)])
@pytest.mark.parametrize("ps", [1, 16])
def test_keys_without_a_valid_slot_are_absent(gpu, dtype, Hq, Hkv, D, ps):
    # table entries outside the pool (page ids, or slots at page size 1) are
    # flagged, never dereferenced, and their keys drop out of the softmax: the
    # outputs equal the oracle over the remaining keys.  Narrow (8/2, 16/4) and
    # wide (32/1) decode items; the extend with invalid keys in stages of pool
    # keys only and in a stage that also holds new tokens.
    g = np.random.default_rng(7 * ps + Hq)
    U = 16  # positions per group below (whole pages when ps = 16)
    S = 8 * U
    n_pages = S // ps
    shape = KVShape(Hq, Hkv, D, DT[dtype], S, ps)
    rnd = lambda *s: (W.round_bf16 if dtype == "bf16" else (lambda x: x))(g.standard_normal(s).astype(np.float32))
    to = lambda a: torch.from_numpy(a).to(gpu).to(DT[dtype])
    kpool, vpool = rnd(S, Hkv, D), rnd(S, Hkv, D)
    # groups of 16 positions: pages (ps = 16) or runs of 16 slots (ps = 1); groups 2 and 4 invalid
    group_ids = [0, 1, n_pages + 3, 2, -5]
    valid = [True, True, False, True, False]
    if ps == 1:
        row = np.concatenate([np.arange(u * U, (u + 1) * U) if ok else np.full(U, x if x < 0 else S + 7)
                              for u, (x, ok) in enumerate(zip(group_ids, valid))]).astype(np.int32)
        slot_of = lambda p: int(row[p])
    else:
        row = np.array(group_ids, np.int32)
        slot_of = lambda p: int(row[p // ps]) * ps + p % ps
    ok_pos = lambda p: valid[p // U]
    tab = np.stack([row, row])
    scale = 1.0 / np.sqrt(D)

    def kv_of(positions):
        sl = [slot_of(p) for p in positions if ok_pos(p)]
        return kpool[sl], vpool[sl]

    err = torch.zeros(1, dtype=torch.int32, device=gpu)
    api.set_error_word(err)
    try:
        # decode: one request over all 80 positions (groups 0..4)
        L = [5 * U]
        q = rnd(1, Hq, D)
        plan = api.plan_decode_unshared(L, Hq // Hkv, 256)
        plan.to(gpu)
        o = torch.empty(1, Hq, D, device=gpu, dtype=DT[dtype])
        ws = torch.empty(api.decode_workspace_bytes(shape, plan), dtype=torch.uint8, device=gpu)
        api.decode_attention(shape, o, to(q), to(kpool), to(vpool), dev(tab, gpu), dev(np.array(L, np.int32), gpu),
                             plan, scale, ws)
        # extend: P = 64 (pool stages only) and P = 40 (its first stage mixes pool keys and new tokens)
        P_list, E_list = [64, 40], [8, 30]
        T = sum(E_list)
        qe, kn, vn = rnd(T, Hq, D), rnd(T, Hkv, D), rnd(T, Hkv, D)
        start = np.array([0, E_list[0]], np.int32)
        ext_o = torch.empty(T, Hq, D, device=gpu, dtype=DT[dtype])
        api.extend_attention(shape, ext_o, to(qe), to(kn), to(vn), to(kpool), to(vpool), dev(tab, gpu),
                             dev(np.array(P_list, np.int32), gpu), dev(np.array(E_list, np.int32), gpu), dev(start, gpu),
                             max(E_list), scale)
        torch.cuda.synchronize()
    finally:
        api.set_error_word(None)
    assert int(err.item()) & 1  # RC_DEVERR_SLOT
    tol = TOL[dtype]
    K, V = kv_of(range(L[0]))
    assert len(K) == 48
    e = float(np.max(np.abs(host(o)[0] - A.decode(q[0], K, V, scale))))
    assert e <= tol, f"decode: max abs error {e:.3e}"
    got = host(ext_o)
    for b, (P, E) in enumerate(zip(P_list, E_list)):
        s0 = int(start[b])
        Kp, Vp = kv_of(range(P))
        want = A.extend(qe[s0:s0 + E], np.concatenate([Kp, kn[s0:s0 + E]]), np.concatenate([Vp, vn[s0:s0 + E]]),
                        len(Kp), scale)
        e = float(np.max(np.abs(got[s0:s0 + E] - want)))
        assert e <= tol, f"extend request {b} (P={P}): max abs error {e:.3e}"


def test_rejects_bad_page_sizes(gpu):
    for ps, S in ((3, 96), (16, 100), (2048, 4096)):
        shape = KVShape(8, 2, 128, torch.bfloat16, S, ps)
        with pytest.raises(Exception):
            api.extend_attention(shape, torch.empty(1, 8, 128, device=gpu, dtype=torch.bfloat16),
                                 torch.empty(1, 8, 128, device=gpu, dtype=torch.bfloat16),
                                 torch.empty(1, 2, 128, device=gpu, dtype=torch.bfloat16),
                                 torch.empty(1, 2, 128, device=gpu, dtype=torch.bfloat16),
                                 torch.empty(S, 2, 128, device=gpu, dtype=torch.bfloat16),
                                 torch.empty(S, 2, 128, device=gpu, dtype=torch.bfloat16),
                                 torch.zeros(1, 4, dtype=torch.int32, device=gpu), torch.zeros(1, dtype=torch.int32, device=gpu),
                                 torch.ones(1, dtype=torch.int32, device=gpu), torch.zeros(1, dtype=torch.int32, device=gpu),
                                 1, 0.1)


# ------------------------------------------------------------- paged workloads
from prefix_shared_kv_amd.engine import Engine  # noqa: E402
from synth import drive  # noqa: E402


def _path_kv(w, nid):
    ids = []
    while nid >= 0:
        ids.append(nid)
        nid = w.nodes[nid].parent
    kv = [w.node_kv(i) for i in reversed(ids)]
    return np.concatenate([k for k, _ in kv]), np.concatenate([v for _, v in kv])


def _queries(w, start, own_q, P, tag):
    """Query rows for positions [P, start + len(own_q)): keyed draws for the recomputed
    tail of the prefix's last partial page, then the workload's own."""
    extra = W.keyed_q(w.seed, w.shape, start - P, 777, tag) if start > P else own_q[:0]
    return np.concatenate([extra, own_q])


def _run_paged(gpu, w, ps, cascade=False, n_steps=None):
    tol = TOL[w.shape.dtype]
    S = (-(-w.pool_slots // ps) + 8 + len(w.requests) + 2 * len(w.nodes)) * ps
    shape = KVShape(w.shape.num_q_heads, w.shape.num_kv_heads, w.shape.head_dim, DT[w.shape.dtype], S, ps)
    longest = max(len(w.prompt_tokens(r)) + r.n_decode + 1 for r in w.requests)
    longest = max([longest] + [w.node_start(n) + len(w.nodes[n].tokens) + 1 for n in range(len(w.nodes))])
    eng = Engine(shape, longest + ps, len(w.requests) + len(w.prefill_nodes) + 2, gpu,
                 free_order=np.random.default_rng(ps).permutation(S // ps).astype(np.int32))
    up = lambda x: drive.up(x, w, gpu)
    worst = 0.0
    # cached nodes: prefill nodes through the extend, the rest stored directly
    for nid in drive.node_order(w):
        toks = drive.path_tokens(w, nid)
        K, V = _path_kv(w, nid)
        start = w.node_start(nid)
        if nid in w.prefill_nodes:
            b = eng.schedule([toks])
            P = int(b.prefix_lens[0])
            assert P % ps == 0 and P <= start
            q = _queries(w, start, w.node_prefill_q(nid), P, nid)
            o = host(eng.extend(b, up(q), up(K[P:]), up(V[P:]), w.sm_scale))
            want = A.extend(q, K, V, P, w.sm_scale)
            e = float(np.max(np.abs(o - want)))
            assert e <= tol, f"prefill node {nid} (P={P}): max abs error {e:.3e}"
            worst = max(worst, e)
            eng.commit(b)
            eng.release(b)
        else:
            m, _ = eng.tree.match(np.concatenate([toks, [-1]]).astype(np.int32))
            assert m % ps == 0 and m <= start
            eng.populate(toks, up(K[m:]), up(V[m:]), expect_cached=m)
    # the requests: prompts extended over their page-rounded cached prefixes
    reqs = w.requests
    reserve = max(r.n_decode for r in reqs)
    b = eng.schedule([w.prompt_tokens(r) for r in reqs], reserve=reserve)
    P = b.prefix_lens
    assert all(p % ps == 0 and p <= len(w.prefix_tokens(r)) for p, r in zip(P, reqs))
    qs, ks, vs, ctx = [], [], [], []
    for i, r in enumerate(reqs):
        K, V = w.context_kv(i, 0)
        pl = len(w.prefix_tokens(r))
        own_q = w.ext_qkv(i)[0]
        qs.append(_queries(w, pl, own_q, int(P[i]), 10000 + i))
        ks.append(K[P[i]:])
        vs.append(V[P[i]:])
        ctx.append((K, V))
    o = host(eng.extend(b, up(np.concatenate(qs)), up(np.concatenate(ks)), up(np.concatenate(vs)), w.sm_scale,
                        cascade=cascade))
    s = 0
    for i in range(len(reqs)):
        want = A.extend(qs[i], ctx[i][0], ctx[i][1], int(P[i]), w.sm_scale)
        e = float(np.max(np.abs(o[s:s + len(qs[i])] - want)))
        assert e <= tol, f"request {i} (P={P[i]}): max abs error {e:.3e}"
        worst = max(worst, e)
        s += len(qs[i])
    eng.commit(b)
    n_steps = reserve if n_steps is None else n_steps
    if n_steps:
        base = [len(w.prompt_tokens(r)) for r in reqs]
        st = eng.prepare_decode(b, base, n_steps, chunk=256)
        rids = list(range(len(reqs)))
        for t in range(n_steps):
            q, k, v = drive.decode_inputs(w, rids, t, device=gpu)
            od = host(eng.decode_step(st, t, q, k, v, w.sm_scale))
            sl = st.slots[t].long()
            assert torch.equal(eng.k_pool[sl], k) and torch.equal(eng.v_pool[sl], v)
            for j in rids:
                K, V = w.context_kv(j, t + 1)
                want = A.decode(w.dec_qkv(j, t)[0], K, V, w.sm_scale)
                e = float(np.max(np.abs(od[j] - want)))
                assert e <= tol, f"decode step {t} request {j}: max abs error {e:.3e}"
                worst = max(worst, e)
    eng.release(b)
    return eng, b, worst


@pytest.mark.parametrize("ps", [16, 64])
def test_paged_gpt2_system_prompt(gpu, ps):
    # 16-token pages: 25 whole pages of the 409-token prompt are shared; each
    # branch recomputes the prompt's last 9 tokens with its own (17 of 417 and
    # 16 of 416 computed, against 8 and 7 at one token per slot)
    w = W.gpt2_system_prompt()
    eng, b, _ = _run_paged(gpu, w, ps, n_steps=8)
    full = (409 // ps) * ps
    assert b.prefix_lens.tolist() == [full, full]
    assert b.extend_lens.tolist() == [417 - full, 416 - full]


@pytest.mark.parametrize("dtype,ps,cascade", [("bf16", 4, False), ("bf16", 16, True), ("f32", 16, False)])
def test_paged_small_tree(gpu, dtype, ps, cascade):
    w = W.multi_turn_tree(depth=3, fanout=3, seg_lo=5, seg_hi=90, ext=9, n_decode=3)
    if dtype == "f32":
        w.shape.dtype = "f32"
    _run_paged(gpu, w, ps, cascade=cascade)
