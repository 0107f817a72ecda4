"""GPU parity on seeded random configurations: head layouts, batch sizes,
prefix and extend lengths (0 and 1 included), page sizes and dtypes drawn per
case.  Extend (tile kernel) and decode with the fused store, through the C ABI,
against the oracle within max-abs 2e-2 (bf16) / 1e-4 (fp32)."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from prefix_shared_kv_amd import KVShape, api
from synth import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DT = {"f32": torch.float32, "bf16": torch.bfloat16}
LAYOUTS = [(4, 4, 64), (8, 2, 128), (32, 8, 128), (32, 4, 128), (12, 12, 64), (16, 1, 64), (24, 3, 128)]


def _case(seed):
    g = np.random.default_rng(1000 + seed)
    Hq, Hkv, D = LAYOUTS[g.integers(len(LAYOUTS))]
    dtype = "f32" if g.random() < 0.3 else "bf16"
    ps = int(g.choice([1, 4, 16]))
    B = int(g.integers(1, 7))
    P = [int(x) for x in g.choice([0, 1, 2, 63, 64, 65, 127, 200, 333], B)]
    E = [int(x) for x in g.choice([0, 1, 7, 31, 32, 33, 64, 130], B)]
    if sum(E) == 0:
        E[0] = 5
    return g, Hq, Hkv, D, dtype, ps, P, E


def _vals(g, dtype, *shape):
    x = g.standard_normal(shape).astype(np.float32)
    return W.round_bf16(x) if dtype == "bf16" else x


@pytest.mark.parametrize("seed", range(16))
def test_random_extend_then_decode(gpu, seed):
    g, Hq, Hkv, D, dtype, ps, P, E = _case(seed)
    dt = DT[dtype]
    B = len(P)
    # each request's context: P cached + E new + 1 decode token, pages drawn in shuffled order
    n_ctx = [p + e + 1 for p, e in zip(P, E)]
    pages = [-(-n // ps) for n in n_ctx]
    n_pages = sum(pages) + 3
    S = n_pages * ps
    order = g.permutation(n_pages).astype(np.int32)
    width = max(pages) + 1
    table = np.full((B + 1, width), -1, np.int32)
    rows = (np.arange(B) + 1).astype(np.int32)
    used = 0
    for b in range(B):
        table[rows[b], :pages[b]] = order[used:used + pages[b]]
        used += pages[b]
    slot = lambda b, p: int(table[rows[b], p // ps]) * ps + p % ps
    K = [_vals(g, dtype, n, Hkv, D) for n in n_ctx]
    V = [_vals(g, dtype, n, Hkv, D) for n in n_ctx]
    kp = np.zeros((S, Hkv, D), np.float32)
    vp = np.zeros((S, Hkv, D), np.float32)
    for b in range(B):
        for p in range(P[b]):
            kp[slot(b, p)], vp[slot(b, p)] = K[b][p], V[b][p]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu).to(dt)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    shape = KVShape(Hq, Hkv, D, dt, S, ps)
    k_pool, v_pool = to(kp), to(vp)
    tab_d = dev(table)
    scale = 1.0 / np.sqrt(D)
    err = torch.zeros(1, dtype=torch.int32, device=gpu)
    api.set_error_word(err)
    try:
        # extend: store the new tokens, then attend
        q = [_vals(g, dtype, e, Hq, D) for e in E]
        start = np.concatenate([[0], np.cumsum(E)[:-1]]).astype(np.int32)
        new_slots = np.array([slot(b, P[b] + i) for b in range(B) for i in range(E[b])], np.int32)
        kn = np.concatenate([K[b][P[b]:P[b] + E[b]] for b in range(B)])
        vn = np.concatenate([V[b][P[b]:P[b] + E[b]] for b in range(B)])
        api.kv_store(shape, k_pool, v_pool, to(kn), to(vn), dev(new_slots))
        o = torch.empty(sum(E), Hq, D, dtype=dt, device=gpu)
        api.extend_attention(shape, o, to(np.concatenate(q)), to(kn), to(vn), k_pool, v_pool, tab_d,
                             dev(np.array(P, np.int32)), dev(np.array(E, np.int32)), dev(start), max(E), scale,
                             rows=dev(rows))
        # decode: one more token per request, stored by the decode call itself
        L = np.array(n_ctx, np.int32)
        qd = _vals(g, dtype, B, Hq, D)
        kd = np.stack([K[b][-1] for b in range(B)])
        vd = np.stack([V[b][-1] for b in range(B)])
        plan = api.plan_decode_unshared(L, Hq // Hkv, int(g.choice([64, 256, 4096])), rows=rows)
        plan.to(gpu)
        od = torch.empty(B, Hq, D, dtype=dt, device=gpu)
        ws = torch.empty(api.decode_workspace_bytes(shape, plan), dtype=torch.uint8, device=gpu)
        api.decode_attention(shape, od, to(qd), k_pool, v_pool, tab_d, dev(L), plan, scale, ws,
                             k_new=to(kd), v_new=to(vd), new_slots=dev(np.array([slot(b, n_ctx[b] - 1) for b in range(B)],
                                                                                 np.int32)))
        torch.cuda.synchronize()
    finally:
        api.set_error_word(None)
    assert int(err.item()) == 0
    got = o.double().cpu().numpy()
    what = f"seed {seed}: {dtype} {Hq}/{Hkv}/{D} page {ps} P={P} E={E}"
    for b in range(B):
        if E[b]:
            want = A.extend(q[b], K[b][:P[b] + E[b]], V[b][:P[b] + E[b]], P[b], scale)
            e = float(np.abs(got[start[b]:start[b] + E[b]] - want).max())
            assert e <= TOL[dtype], f"{what}: extend request {b} error {e:.3e}"
    gd = od.double().cpu().numpy()
    for b in range(B):
        want = A.decode(qd[b], K[b], V[b], scale)
        e = float(np.abs(gd[b] - want).max())
        assert e <= TOL[dtype], f"{what}: decode request {b} error {e:.3e}"
