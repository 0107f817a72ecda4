"""GPU invariants that hold whatever the values, checked through the engine
(every call through the C ABI) on whole workloads:

- softmax weights sum to one: with V = 1 everywhere, every bf16 output of the
  extend (tile and cascade), the prefill and every decode step is exactly 1.0
  (P is rounded to bf16 once and the same rounded weights give numerator and
  denominator, so the quotient is 1 to fp32 rounding, which bf16 cannot show);
- slot numbering does not enter the arithmetic: the same workload over a pool
  handed out in identity order and in a shuffled order gives bit-identical
  outputs;
- node boundaries do not either: a sequence cut anywhere into cached prefix and
  new tokens gives the tile extend's outputs bit for bit (its key stages are
  aligned to absolute position 0).
"""
import numpy as np
import pytest
import torch

from synth import drive
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _small_tree():
    # depth 3, fanout 3: the root's children are shared by 9 requests (wide
    # decode items at GQA 32/8), their children by 3 (narrow ones)
    return W.multi_turn_tree(depth=3, fanout=3, seg_lo=5, seg_hi=90, ext=9, n_decode=3)


def _ones_v(w):
    orig = w._vals

    def vals(shape, tag, *ids):
        x = orig(shape, tag, *ids)
        return np.ones_like(x) if tag in (W._T_NODE_V, W._T_EXT_V, W._T_DEC_V) else x

    w._vals = vals
    return w


def _run(gpu, w, cascade, n_steps):
    """Every output of the workload: prefill nodes, the requests' extend, n_steps decode steps."""
    eng = drive.make_engine(w, gpu)
    drive.populate(eng, w, [n for n in drive.node_order(w) if n not in w.prefill_nodes], device=gpu)
    outs = [o.clone() for o in drive.prefill_nodes(eng, w, gpu).values()]
    b, o = drive.extend_requests(eng, w, device=gpu, cascade=cascade)
    outs.append(o.clone())
    base = [len(w.prompt_tokens(r)) for r in w.requests]
    st = eng.prepare_decode(b, base, n_steps, chunk=64)
    rids = list(range(len(w.requests)))
    for t in range(n_steps):
        q, k, v = drive.decode_inputs(w, rids, t, device=gpu)
        outs.append(eng.decode_step(st, t, q, k, v, w.sm_scale).clone())
    eng.release(b)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("name,cascade", [("gpt2", False), ("gpt2", True), ("tree", False), ("tree", True)])
def test_unit_values_give_exactly_one(gpu, name, cascade):
    w = _ones_v(W.gpt2_system_prompt() if name == "gpt2" else _small_tree())
    outs = _run(gpu, w, cascade, 3)
    for i, o in enumerate(outs):
        assert o.dtype == torch.bfloat16
        bad = (o != 1).sum().item()
        assert bad == 0, f"output {i}: {bad} of {o.numel()} elements differ from 1 (max |o-1| {(o.float() - 1).abs().max().item():.3e})"


@pytest.mark.parametrize("name,cascade", [("gpt2", False), ("tree", True)])
def test_slot_order_does_not_change_any_bit(gpu, name, cascade):
    runs = []
    for shuffled in (False, True):
        w = W.gpt2_system_prompt() if name == "gpt2" else _small_tree()
        w.shuffle_slots = shuffled
        runs.append(_run(gpu, w, cascade, 3))
    for i, (a, b) in enumerate(zip(*runs)):
        assert torch.equal(a, b), f"output {i} differs between slot orders"


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 32, 8, 128), ("bf16", 12, 12, 64), ("f32", 8, 2, 64)])
def test_any_cached_length_gives_the_same_bits(gpu, dtype, Hq, Hkv, D):
    # One logical sequence of N tokens, cut at P' cached + N - P' new tokens for
    # several P' in one batch.  The tile walks keys in stages aligned to
    # absolute position 0, so the outputs of positions >= P (every cut <= P)
    # are bit-identical whatever P' is, and match the oracle.
    from oracle import attention as A
    from prefix_shared_kv_amd import KVShape, api
    N, P = 300, 200
    cuts = [0, 1, 63, 64, 65, 128, 199, 200]
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    g = np.random.default_rng(Hq * D)
    rnd = lambda *s: (W.round_bf16 if dtype == "bf16" else (lambda x: x))(g.standard_normal(s).astype(np.float32))
    q, k, v = rnd(N, Hq, D), rnd(N, Hkv, D), rnd(N, Hkv, D)
    S = N + 64
    slots = g.permutation(S)[:N].astype(np.int32)
    kp = torch.zeros(S, Hkv, D, dtype=dt, device=gpu)
    vp = torch.zeros_like(kp)
    kp[torch.from_numpy(slots.astype(np.int64)).to(gpu)] = torch.from_numpy(k).to(gpu).to(dt)
    vp[torch.from_numpy(slots.astype(np.int64)).to(gpu)] = torch.from_numpy(v).to(gpu).to(dt)
    B = len(cuts)
    table = np.tile(slots, (B, 1))
    E = [N - c for c in cuts]
    start = np.concatenate([[0], np.cumsum(E)[:-1]]).astype(np.int32)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu).to(dt)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    qs = np.concatenate([q[c:] for c in cuts])
    ks = np.concatenate([k[c:] for c in cuts])
    vs = np.concatenate([v[c:] for c in cuts])
    o = torch.empty(len(qs), Hq, D, dtype=dt, device=gpu)
    shape = KVShape(Hq, Hkv, D, dt, S)
    api.extend_attention(shape, o, to(qs), to(ks), to(vs), kp, vp, dev(table), dev(np.array(cuts, np.int32)),
                         dev(np.array(E, np.int32)), dev(start), max(E), 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    tail = [o[start[b] + (P - cuts[b]):start[b] + E[b]] for b in range(B)]
    for b in range(1, B):
        assert torch.equal(tail[b], tail[0]), f"cut {cuts[b]} differs from cut {cuts[0]}"
    want = A.extend(q[P:], k, v, P, 1.0 / np.sqrt(D))
    err = float((tail[0].double().cpu() - torch.from_numpy(want)).abs().max())
    assert err <= {"bf16": 2e-2, "f32": 1e-4}[dtype], err


def test_batches_rescheduled_on_their_own_rows(gpu):
    # caller-owned rows (take_rows): the same requests, then a permuted order
    # (rows rewritten from their first entries), then the same again; only the
    # entries a schedule changes are uploaded, and every extend still matches
    # the oracle
    from oracle import attention as A
    w = _small_tree()
    eng = drive.make_engine(w, gpu, max_rows=2 * len(w.requests) + 4)
    drive.populate(eng, w, device=gpu)
    n = len(w.requests)
    rows = eng.take_rows(n)
    for order in (np.arange(n), np.random.default_rng(0).permutation(n), np.arange(n)):
        b = eng.schedule([w.prompt_tokens(w.requests[i]) for i in order], reserve=2, rows=rows)
        assert b.prefix_lens.tolist() == [len(w.prefix_tokens(w.requests[i])) for i in order]
        qs, ks, vs = zip(*(w.ext_qkv(int(i)) for i in order))
        o = eng.extend(b, *(drive.up(np.concatenate(x), w, gpu) for x in (qs, ks, vs)), w.sm_scale)
        got = o.float().cpu().numpy()
        s = 0
        for j, i in enumerate(order):
            K, V = w.context_kv(int(i), 0)
            want = A.extend(qs[j], K, V, int(b.prefix_lens[j]), w.sm_scale)
            err = float(np.abs(got[s:s + len(qs[j])] - want).max())
            assert err <= 2e-2, (j, err)
            s += len(qs[j])
        eng.release(b, keep=b.prefix_lens)
    eng.give_rows(rows)
    assert len(eng.free_rows) == 2 * len(w.requests) + 4
