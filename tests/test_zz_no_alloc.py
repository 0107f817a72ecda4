"""The allocation-free decode entry point (rc_decode_attention_static) against
rc_decode_attention.  Both run the same kernels; the first writes its partials
to a static per-GPU workspace inside the library, the second to the caller's.
So their outputs must be bit-identical, and both must match the oracle
(max-abs 2e-2 for bf16, 1e-4 for fp32).

Two calls in a row on one GPU, the second with a smaller batch, because the
static workspace keeps the first call's contents.  A plan whose workspace
exceeds the static size is rejected before anything is launched."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from prefix_shared_kv_amd import _native as N
from prefix_shared_kv_amd import KVShape, api
from synth import drive
from synth import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def decode_both_ways(gpu, w, chunk):
    """One decode step of every request of w, through both entry points; returns the max
    abs error of the static call's outputs against the oracle."""
    eng = drive.make_engine(w, device=gpu)
    drive.prefill_nodes(eng, w, device=gpu)
    rest = [n for n in drive.node_order(w) if n not in w.prefill_nodes]
    drive.populate(eng, w, rest, device=gpu)
    b, _ = drive.extend_requests(eng, w, device=gpu)
    B = len(w.requests)
    base = [len(w.prompt_tokens(r)) for r in w.requests]
    st = eng.prepare_decode(b, base, 1, chunk=chunk)
    assert api.decode_workspace_bytes(eng.shape, st.plan) <= N.RC_DECODE_STATIC_WORKSPACE_BYTES
    q, k, v = drive.decode_inputs(w, range(B), 0, device=gpu)
    o_ref = torch.full_like(q, 3.0)
    o_static = torch.full_like(q, -3.0)
    # both calls store the step's K/V into the same slots (the same bits) and read them back
    api.decode_attention(eng.shape, o_ref, q, eng.k_pool, eng.v_pool, eng.table_d, st.seq_lens[0], st.plan,
                         w.sm_scale, st.workspace, k_new=k, v_new=v, new_slots=st.slots[0])
    api.decode_attention_static(eng.shape, o_static, q, eng.k_pool, eng.v_pool, eng.table_d, st.seq_lens[0], st.plan,
                                w.sm_scale, k_new=k, v_new=v, new_slots=st.slots[0])
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o_static), "static-workspace decode differs from the caller-workspace decode"
    got = host(o_static)
    worst = 0.0
    for i in range(B):
        K, V = w.context_kv(i, 1)
        want = A.decode(w.dec_qkv(i, 0)[0], K, V, w.sm_scale)
        e = float(np.max(np.abs(got[i] - want)))
        assert e <= TOL[w.shape.dtype], f"request {i}: max abs error {e:.3e}"
        worst = max(worst, e)
    return worst


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_static_workspace_decode_twice_second_smaller(gpu, dtype):
    # a nested tree of 27 requests with many splits (pieces of 32 positions),
    # then 3 requests of a few-shot batch: the second call reads only the
    # partials it wrote, whatever the first left in the shared workspace
    big = W.multi_turn_tree(depth=3, fanout=3, seg_lo=20, seg_hi=120, ext=7, n_decode=1)
    small = W.few_shot(n_req=3, prefix=150, ext=5, n_decode=1)
    for w in (big, small):
        if dtype == "f32":
            w.shape.dtype = "f32"
    decode_both_ways(gpu, big, chunk=32)
    decode_both_ways(gpu, small, chunk=4096)


def test_static_workspace_rejects_plans_too_large(gpu):
    # 1024 requests x 32 heads x 9 splits x (128 bf16 + 2 fp32) = 77.9 MB > 64 MiB
    B, Hq, Hkv, D = 1024, 32, 8, 128
    shape = KVShape(Hq, Hkv, D, torch.bfloat16, 64)
    plan = api.plan_decode_unshared(np.full(B, 640, np.int32), Hq // Hkv, 64)
    assert api.decode_workspace_bytes(shape, plan) > N.RC_DECODE_STATIC_WORKSPACE_BYTES
    plan.to(gpu)
    q = torch.zeros(B, Hq, D, device=gpu, dtype=torch.bfloat16)
    o = torch.full_like(q, 5.0)
    pool = torch.zeros(64, Hkv, D, device=gpu, dtype=torch.bfloat16)
    table = torch.zeros(B, 640, dtype=torch.int32, device=gpu)
    seq = torch.full((B,), 640, dtype=torch.int32, device=gpu)
    with pytest.raises(N.RcError) as e:
        api.decode_attention_static(shape, o, q, pool, pool, table, seq, plan, 0.1)
    assert e.value.status == N.RC_ERR_RANGE and "static workspace" in str(e.value)
    torch.cuda.synchronize()
    assert bool((o == 5.0).all())  # nothing was launched
