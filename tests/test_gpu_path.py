"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: KV scatter bit-exact over the whole pool; attention within max-abs 1e-4
for fp32 inputs and 2e-2 for bf16 inputs of the float64 oracle."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from prefix_shared_kv_amd import KVShape, api
from synth import drive
from synth import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(got, want, tol, what):
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol}"
    return err


# ---------------------------------------------------------------- KV scatter
@pytest.mark.parametrize("dtype,H,D", [("bf16", 8, 128), ("f32", 4, 64), ("bf16", 12, 64)])
def test_kv_store_bit_exact_whole_pool(gpu, dtype, H, D):
    S, n = 1000, 333
    g = np.random.default_rng(0)
    shape = KVShape(H, H, D, DT[dtype], S)
    pool_k = torch.randn(S, H, D, device=gpu).to(DT[dtype])
    pool_v = torch.randn(S, H, D, device=gpu).to(DT[dtype])
    new_k = torch.randn(n, H, D, device=gpu).to(DT[dtype])
    new_v = torch.randn(n, H, D, device=gpu).to(DT[dtype])
    slots = g.choice(S, n, replace=False).astype(np.int32)
    ibits = torch.int16 if dtype == "bf16" else torch.int32
    before_k, before_v = pool_k.view(ibits).cpu().numpy(), pool_v.view(ibits).cpu().numpy()
    api.kv_store(shape, pool_k, pool_v, new_k, new_v, torch.from_numpy(slots).to(gpu))
    torch.cuda.synchronize()
    want_k = A.kv_store(before_k, new_k.view(ibits).cpu().numpy(), slots)
    want_v = A.kv_store(before_v, new_v.view(ibits).cpu().numpy(), slots)
    assert np.array_equal(pool_k.view(ibits).cpu().numpy(), want_k)
    assert np.array_equal(pool_v.view(ibits).cpu().numpy(), want_v)


def test_kv_store_flags_out_of_range_slot(gpu):
    shape = KVShape(2, 2, 64, torch.bfloat16, 8)
    pool = torch.zeros(8, 2, 64, device=gpu, dtype=torch.bfloat16)
    pool_v = torch.zeros_like(pool)
    new = torch.ones(2, 2, 64, device=gpu, dtype=torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device=gpu)
    api.set_error_word(err)
    try:
        api.kv_store(shape, pool, pool_v, new, new, torch.tensor([3, 8], dtype=torch.int32, device=gpu))
        torch.cuda.synchronize()
    finally:
        api.set_error_word(None)
    assert int(err.item()) & 1
    assert float(pool[3].float().sum()) == 128.0 and float(pool.float().sum()) == 128.0


# ---------------------------------------------------------------- extend, direct API
def _extend_case(gpu, dtype, Hq, Hkv, D, P_list, E_list, seed=0, shuffled=True):
    g = np.random.default_rng(seed)
    B = len(P_list)
    S = sum(P_list) + 64
    shape = KVShape(Hq, Hkv, D, DT[dtype], S)
    std = 1.0

    def rnd(*s):
        x = g.standard_normal(s).astype(np.float32) * std
        return W.round_bf16(x) if dtype == "bf16" else x

    pk = [rnd(p, Hkv, D) for p in P_list]
    pv = [rnd(p, Hkv, D) for p in P_list]
    T = sum(E_list)
    q, kn, vn = rnd(T, Hq, D), rnd(T, Hkv, D), rnd(T, Hkv, D)
    order = g.permutation(S).astype(np.int32) if shuffled else np.arange(S, dtype=np.int32)
    stride = max(P_list) + 3
    table = np.full((B + 2, stride), -1, np.int32)
    pool_k = torch.zeros(S, Hkv, D, device=gpu, dtype=DT[dtype])
    pool_v = torch.zeros_like(pool_k)
    used = 0
    rows = (np.arange(B) + 1).astype(np.int32)  # not the identity mapping
    for b, p in enumerate(P_list):
        sl = order[used:used + p]
        used += p
        table[rows[b], :p] = sl
        if p:
            idx = torch.from_numpy(sl.astype(np.int64)).to(gpu)
            pool_k[idx] = torch.from_numpy(pk[b]).to(gpu).to(DT[dtype])
            pool_v[idx] = torch.from_numpy(pv[b]).to(gpu).to(DT[dtype])
    start = np.concatenate([[0], np.cumsum(E_list)[:-1]]).astype(np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    to = lambda a: torch.from_numpy(a).to(gpu).to(DT[dtype])
    o = torch.full((T, Hq, D), 7.0, device=gpu, dtype=DT[dtype])
    err = torch.zeros(1, dtype=torch.int32, device=gpu)
    api.set_error_word(err)
    try:
        api.extend_attention(shape, o, to(q), to(kn), to(vn), pool_k, pool_v, dev(table),
                             dev(np.array(P_list, np.int32)), dev(np.array(E_list, np.int32)), dev(start),
                             max(E_list) if E_list else 0, 1.0 / np.sqrt(D), rows=dev(rows))
        torch.cuda.synchronize()
    finally:
        api.set_error_word(None)
    assert int(err.item()) == 0
    got = host(o)
    worst = 0.0
    for b in range(B):
        E = E_list[b]
        if E == 0:
            continue
        s0 = start[b]
        K = np.concatenate([pk[b], kn[s0:s0 + E]])
        V = np.concatenate([pv[b], vn[s0:s0 + E]])
        want = A.extend(q[s0:s0 + E], K, V, P_list[b], 1.0 / np.sqrt(D))
        worst = max(worst, check(got[s0:s0 + E], want, TOL[dtype], f"request {b} (P={P_list[b]}, E={E})"))
    return worst


# group sizes 1 to 128 (the largest the library accepts): with 32 and more
# query heads per kv head an extend tile holds 256 / group tokens
HEAD_LAYOUTS = [(4, 4, 64), (8, 2, 128), (32, 8, 128), (16, 1, 64), (12, 4, 128), (24, 3, 64),
                (32, 1, 128), (64, 1, 128), (128, 1, 64), (64, 2, 64)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv,D", HEAD_LAYOUTS)
def test_extend_ragged_against_oracle(gpu, dtype, Hq, Hkv, D):
    P_list = [0, 1, 63, 64, 130, 300, 5]
    E_list = [70, 1, 65, 0, 33, 129, 8]
    _extend_case(gpu, dtype, Hq, Hkv, D, P_list, E_list, seed=Hq * 100 + D)


def test_extend_single_token_prefill_is_value(gpu):
    # first token of an empty-prefix prefill sees only itself: o = v (after bf16 rounding of v: exact)
    _extend_case(gpu, "bf16", 8, 8, 128, [0], [1])


# ---------------------------------------------------------------- whole workloads
def _run_workload(gpu, w, shared=True, chunk=512, decode_steps=None, fused=True, cascade=False):
    tol = TOL[w.shape.dtype]
    eng = drive.make_engine(w, device=gpu)
    errs = []
    outs = drive.prefill_nodes(eng, w, device=gpu)
    for nid, o in outs.items():
        k, v = w.node_kv(nid)
        want = A.extend(w.node_prefill_q(nid), k, v, 0, w.sm_scale)
        errs.append(check(host(o), want, tol, f"prefill node {nid}"))
    rest = [n for n in drive.node_order(w) if n not in w.prefill_nodes]
    drive.populate(eng, w, rest, device=gpu)
    rids = list(range(len(w.requests)))
    has_ext = any(len(r.ext_tokens) for r in w.requests)
    if has_ext:
        b, o = drive.extend_requests(eng, w, rids, device=gpu, cascade=cascade)
        got = host(o)
        s = 0
        for i in rids:
            q, _, _ = w.ext_qkv(i)
            K, V = w.context_kv(i, 0)
            P = len(w.prefix_tokens(w.requests[i]))
            want = A.extend(q, K, V, P, w.sm_scale)
            errs.append(check(got[s:s + len(q)], want, tol, f"extend request {i}"))
            s += len(q)
        base = [len(w.prompt_tokens(w.requests[i])) for i in rids]
    else:
        b = drive.schedule_decode_only(eng, w, rids)
        base = [len(w.prompt_tokens(w.requests[i])) for i in rids]
    n_steps = decode_steps if decode_steps is not None else max(r.n_decode for r in w.requests)
    if n_steps:
        st = eng.prepare_decode(b, base, n_steps, chunk=chunk, shared=shared)
        for t in range(n_steps):
            q, k, v = drive.decode_inputs(w, rids, t, device=gpu)
            o = host(eng.decode_step(st, t, q, k, v, w.sm_scale, fused_store=fused))
            # the step's K/V landed in the pool, bit for bit
            sl = st.slots[t].long()
            assert torch.equal(eng.k_pool[sl], k) and torch.equal(eng.v_pool[sl], v)
            for j, i in enumerate(rids):
                K, V = w.context_kv(i, t + 1)
                want = A.decode(w.dec_qkv(i, t)[0], K, V, w.sm_scale)
                errs.append(check(o[j], want, tol, f"decode step {t} request {i}"))
    return eng, b, max(errs)


@pytest.mark.parametrize("fused", [True, False])
def test_tiny_fp32_workload(gpu, fused):
    _run_workload(gpu, W.tiny_fp32(), fused=fused)


@pytest.mark.parametrize("shared,chunk,fused", [(True, 512, True), (False, 512, True), (True, 64, False),
                                                (False, 4096, False)])
def test_gpt2_system_prompt_workload(gpu, shared, chunk, fused):
    w = W.gpt2_system_prompt()
    eng, b, err = _run_workload(gpu, w, shared=shared, chunk=chunk, fused=fused)
    # the glossary's bookkeeping: 8 of 417 and 7 of 416 tokens computed
    assert [(int(e), int(p + e)) for p, e in zip(b.prefix_lens, b.extend_lens)] == [(8, 417), (7, 416)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_radix_tree_workload_shared_vs_unshared(gpu, dtype):
    w = W.multi_turn_tree(depth=3, fanout=3, seg_lo=5, seg_hi=90, ext=9, n_decode=3)
    if dtype == "f32":
        w.shape.dtype = "f32"
    for shared, chunk in [(True, 32), (True, 4096), (False, 64)]:
        _run_workload(gpu, w, shared=shared, chunk=chunk)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cascade_extend_matches_the_oracle(gpu, dtype):
    # new tokens through the shared-prefix plan (split-K kernel + merge):
    # a nested tree, branches over one document, and the GPT-2 system prompt
    for w in (W.multi_turn_tree(depth=3, fanout=3, seg_lo=5, seg_hi=90, ext=9, n_decode=2),
              W.classify64(prefix=300, n_branch=12), W.gpt2_system_prompt()):
        if dtype == "f32":
            w.shape.dtype = "f32"
        _run_workload(gpu, w, cascade=True, decode_steps=0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 1, 128), (64, 1, 128), (128, 1, 64)])
def test_cascade_extend_large_groups(gpu, dtype, Hq, Hkv, D):
    # branches over one document through the shared-prefix plan with 32 to 128
    # query heads per kv head (8 to 2 new tokens per 256-column member group)
    w = W.classify64(prefix=300, n_branch=12)
    w.shape.num_q_heads, w.shape.num_kv_heads, w.shape.head_dim = Hq, Hkv, D
    w.sm_scale = 1.0 / np.sqrt(D)
    if dtype == "f32":
        w.shape.dtype = "f32"
    _run_workload(gpu, w, cascade=True, decode_steps=0)


def test_decode_is_deterministic(gpu):
    w = W.few_shot(n_req=6, prefix=200, ext=5, n_decode=2)
    outs = []
    for _ in range(2):
        eng = drive.make_engine(w, device=gpu)
        drive.prefill_nodes(eng, w, device=gpu)
        b, o = drive.extend_requests(eng, w, device=gpu)
        st = eng.prepare_decode(b, [len(w.prompt_tokens(r)) for r in w.requests], 2, chunk=64)
        q, k, v = drive.decode_inputs(w, range(6), 0, device=gpu)
        d = eng.decode_step(st, 0, q, k, v, w.sm_scale)
        outs.append((o.view(torch.int16).cpu(), d.view(torch.int16).cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_decode_launcher_equals_the_plain_call(gpu):
    # the engine's per-batch launcher (fixed arguments checked once) gives the
    # bits of rc_decode_attention called through api.decode_attention, pool
    # writes included, and rejects a step tensor of the wrong shape or dtype
    w = W.few_shot(n_req=6, prefix=200, ext=5, n_decode=3)
    res = []
    for plain in (False, True):
        eng = drive.make_engine(w, device=gpu)
        drive.prefill_nodes(eng, w, device=gpu)
        b, _ = drive.extend_requests(eng, w, device=gpu)
        st = eng.prepare_decode(b, [len(w.prompt_tokens(r)) for r in w.requests], 3, chunk=64)
        outs = []
        for t in range(3):
            q, k, v = drive.decode_inputs(w, range(6), t, device=gpu)
            if plain:
                o = torch.empty_like(q)
                api.decode_attention(eng.shape, o, q, eng.k_pool, eng.v_pool, eng.table_d, st.seq_lens[t], st.plan,
                                     w.sm_scale, st.workspace, k_new=k, v_new=v, new_slots=st.slots[t])
            else:
                o = eng.decode_step(st, t, q, k, v, w.sm_scale)
            outs.append(o.view(torch.int16).cpu())
        sl = st.slots.long().reshape(-1)
        res.append((outs, eng.k_pool[sl].view(torch.int16).cpu(), eng.v_pool[sl].view(torch.int16).cpu()))
        if not plain:
            q, k, v = drive.decode_inputs(w, range(6), 0, device=gpu)
            with pytest.raises(ValueError):
                eng.decode_step(st, 0, q[:5], k, v, w.sm_scale)
            with pytest.raises(ValueError):
                eng.decode_step(st, 0, q.float(), k, v, w.sm_scale)
            with pytest.raises(IndexError):
                eng.decode_step(st, 3, q, k, v, w.sm_scale)
    assert all(torch.equal(x, y) for x, y in zip(res[0][0], res[1][0]))
    assert torch.equal(res[0][1], res[1][1]) and torch.equal(res[0][2], res[1][2])


def test_unused_pool_slots_holding_nan_do_not_leak(gpu):
    # past-the-end keys of a stage read some pool row; its contents must never reach the output
    w = W.multi_turn_tree(depth=2, fanout=3, seg_lo=7, seg_hi=70, ext=5, n_decode=2)
    eng = drive.make_engine(w, device=gpu)
    eng.k_pool.fill_(float("nan"))
    eng.v_pool.fill_(float("nan"))
    drive.populate(eng, w, device=gpu)
    b, o = drive.extend_requests(eng, w, device=gpu)
    assert torch.isfinite(o.float()).all()
    st = eng.prepare_decode(b, [len(w.prompt_tokens(r)) for r in w.requests], 2, chunk=48)
    for t in range(2):
        q, k, v = drive.decode_inputs(w, range(len(w.requests)), t, device=gpu)
        d = host(eng.decode_step(st, t, q, k, v, w.sm_scale))
        for i in range(len(w.requests)):
            K, V = w.context_kv(i, t + 1)
            check(d[i], A.decode(w.dec_qkv(i, t)[0], K, V, w.sm_scale), TOL["bf16"], f"decode step {t} request {i}")


@pytest.mark.parametrize("Hq,Hkv,D", [(12, 3, 128), (16, 2, 64), (8, 8, 128), (48, 12, 64),
                                      (32, 1, 128), (64, 1, 128), (128, 1, 64), (64, 2, 64)])
def test_decode_head_layouts(gpu, Hq, Hkv, D):
    # wide and narrow decode items over shared and unshared plans (groups of 32
    # and more make every item wide: 128 / group members per item)
    w = W.multi_turn_tree(depth=3, fanout=2, seg_lo=20, seg_hi=150, ext=6, n_decode=2)
    w.shape.num_q_heads, w.shape.num_kv_heads, w.shape.head_dim = Hq, Hkv, D
    w.sm_scale = 1.0 / np.sqrt(D)
    for shared, chunk in [(True, 64), (False, 100)]:
        _run_workload(gpu, w, shared=shared, chunk=chunk)


@pytest.mark.parametrize("prefix,dtype,D", [(1500, "bf16", 128), (256, "bf16", 128), (272, "bf16", 128),
                                             (272, "f32", 64), (272, "bf16", 64)])
def test_decode_merge_of_many_splits(gpu, prefix, dtype, D):
    # the merge combines the partials 16 splits at a time: 85 splits over a
    # 1500-token prefix (six blocks, each rescaled against the next), and 16
    # and 17 splits (the shared prefix in 15 or 16 pieces of at most 18
    # positions, plus each request's own range) on both sides of one block;
    # fp32 partial rows and head_dim 64 take their own loads
    w = W.few_shot(n_req=3, prefix=prefix, ext=5, n_decode=1)
    w.shape.dtype, w.shape.head_dim = dtype, D
    w.sm_scale = 1.0 / np.sqrt(D)
    _run_workload(gpu, w, shared=True, chunk=16)
