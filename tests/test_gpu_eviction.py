"""GPU parity under LRU eviction: four chat sessions run through a pool that
holds about two of them.  Prefixes are reused, evicted and recomputed; every
extend and decode output must still equal the oracle's attention over the
request's whole logical context (K/V at a position depend only on the tokens
up to it), and the engine's prefix lengths and evictions must be those of the
plain LRU tree model."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.lru_tree import LruTree
from prefix_shared_kv_amd import KVShape
from prefix_shared_kv_amd.engine import Engine
from synth import workloads as W

pytestmark = pytest.mark.gpu

TOL = 2e-2
SEED = 17
SH = W.Shape(32, 8, 128, "bf16")
POOL = 1288


def sessions():
    g = np.random.default_rng(0)
    first = [[1000 * s + 1] + [int(x) for x in g.integers(0, 50000, 383)] for s in range(4)]
    turn = {(s, j): [int(x) for x in g.integers(0, 50000, 96)] for s in range(4) for j in range(3)}
    return [([first[0]], 0), ([first[1]], 0), ([first[2]], 0), ([first[3]], 0),
            ([first[0] + turn[0, 0]], 0), ([first[3] + turn[3, 0]], 0),
            ([first[0] + turn[0, 0] + turn[0, 1], first[1] + turn[1, 0]], 2)]


def dev(a, gpu):
    return torch.from_numpy(np.ascontiguousarray(a)).to(gpu).to(torch.bfloat16)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_sessions_through_a_small_pool(gpu):
    reqs = sessions()
    shape = KVShape(SH.num_q_heads, SH.num_kv_heads, SH.head_dim, torch.bfloat16, POOL)
    eng = Engine(shape, stride=1024, max_rows=8, device=gpu)
    model = LruTree(POOL)
    scale = 1.0 / np.sqrt(SH.head_dim)
    n_steps = 2
    for i, (batch, reserve) in enumerate(reqs):
        print(f"request {i}: lengths {[len(t) for t in batch]}, reserve {reserve}", flush=True)
        rows_m, P_m, _, locks_m = model.emit_rows(batch, reserve=reserve, evict=True, lock=True)
        ev_before = eng.tree.stats()["evicted_tokens"]
        b = eng.schedule(batch, reserve=reserve)
        assert b.prefix_lens.tolist() == P_m, f"request {i}"
        assert eng.tree.stats()["evicted_tokens"] == model.evicted_tokens, f"request {i}"
        P = b.prefix_lens
        kv = [W.prefix_keyed_kv(SEED, np.array(t + [50257 + s for s in range(reserve)]), SH) for t in batch]
        q = [W.keyed_q(SEED, SH, len(t), i, j) for j, t in enumerate(batch)]
        qn = np.concatenate([q[j][P[j]:] for j in range(len(batch))])
        kn = np.concatenate([kv[j][0][P[j]:len(t)] for j, t in enumerate(batch)])
        vn = np.concatenate([kv[j][1][P[j]:len(t)] for j, t in enumerate(batch)])
        o = host(eng.extend(b, dev(qn, gpu), dev(kn, gpu), dev(vn, gpu), scale))
        off = 0
        for j, t in enumerate(batch):
            e = len(t) - P[j]
            want = A.extend(q[j][P[j]:], kv[j][0][:len(t)], kv[j][1][:len(t)], int(P[j]), scale)
            err = float(np.max(np.abs(o[off:off + e] - want)))
            assert err <= TOL, f"request {i}.{j} extend (P={P[j]}): max abs error {err:.3e}"
            off += e
        eng.commit(b)
        for r, row in zip(batch, rows_m):
            model.insert(r, row[:len(r)])
        if reserve:
            base = [len(t) for t in batch]
            st = eng.prepare_decode(b, base, n_steps)
            for s in range(n_steps):
                qd = np.stack([W.keyed_q(SEED, SH, 1, 100 + i, j, s)[0] for j in range(len(batch))])
                kd = np.stack([kv[j][0][base[j] + s] for j in range(len(batch))])
                vd = np.stack([kv[j][1][base[j] + s] for j in range(len(batch))])
                od = host(eng.decode_step(st, s, dev(qd, gpu), dev(kd, gpu), dev(vd, gpu), scale))
                for j in range(len(batch)):
                    n = base[j] + s + 1
                    want = A.decode(qd[j], kv[j][0][:n], kv[j][1][:n], scale)
                    err = float(np.max(np.abs(od[j] - want)))
                    assert err <= TOL, f"request {i}.{j} decode step {s}: max abs error {err:.3e}"
        eng.release(b)
        for lid in locks_m:
            model.unlock(lid)
        for r, row in zip(batch, rows_m):
            model.free_slots(row[len(r):])
        st_n, st_m = eng.tree.stats(), model.stats()
        for k in ("nodes", "cached_tokens", "free_slots", "evicted_tokens", "locked_tokens"):
            assert st_n[k] == st_m[k], f"request {i}: {k}"
    # the run reused a prefix, recomputed one that was evicted, and evicted while a batch ran
    assert eng.tree.stats()["evicted_tokens"] >= 1000


@pytest.mark.parametrize("ps", [16, 64])
def test_sessions_through_a_small_paged_pool(gpu, ps):
    # the same sessions over a pool of pages: the tree stores, shares and evicts
    # whole pages; every output must still be the oracle's attention over the
    # request's logical context, and prefixes must be reused (in whole pages)
    # and evicted along the way
    reqs = sessions()
    n_pages = -(-POOL // ps)
    shape = KVShape(SH.num_q_heads, SH.num_kv_heads, SH.head_dim, torch.bfloat16, n_pages * ps, ps)
    eng = Engine(shape, stride=1024, max_rows=8, device=gpu)
    scale = 1.0 / np.sqrt(SH.head_dim)
    n_steps = 2
    reused = 0
    for i, (batch, reserve) in enumerate(reqs):
        print(f"request {i}: lengths {[len(t) for t in batch]}, reserve {reserve}, page {ps}", flush=True)
        b = eng.schedule(batch, reserve=reserve)
        P = b.prefix_lens
        assert all(p % ps == 0 and p < len(t) for p, t in zip(P, batch)), f"request {i}"
        reused += int(P.sum())
        kv = [W.prefix_keyed_kv(SEED, np.array(t + [50257 + s for s in range(reserve)]), SH) for t in batch]
        q = [W.keyed_q(SEED, SH, len(t), i, j) for j, t in enumerate(batch)]
        qn = np.concatenate([q[j][P[j]:] for j in range(len(batch))])
        kn = np.concatenate([kv[j][0][P[j]:len(t)] for j, t in enumerate(batch)])
        vn = np.concatenate([kv[j][1][P[j]:len(t)] for j, t in enumerate(batch)])
        o = host(eng.extend(b, dev(qn, gpu), dev(kn, gpu), dev(vn, gpu), scale))
        off = 0
        for j, t in enumerate(batch):
            e = len(t) - P[j]
            want = A.extend(q[j][P[j]:], kv[j][0][:len(t)], kv[j][1][:len(t)], int(P[j]), scale)
            err = float(np.max(np.abs(o[off:off + e] - want)))
            assert err <= TOL, f"request {i}.{j} extend (P={P[j]}): max abs error {err:.3e}"
            off += e
        eng.commit(b)
        if reserve:
            base = [len(t) for t in batch]
            st = eng.prepare_decode(b, base, n_steps)
            for s in range(n_steps):
                qd = np.stack([W.keyed_q(SEED, SH, 1, 100 + i, j, s)[0] for j in range(len(batch))])
                kd = np.stack([kv[j][0][base[j] + s] for j in range(len(batch))])
                vd = np.stack([kv[j][1][base[j] + s] for j in range(len(batch))])
                od = host(eng.decode_step(st, s, dev(qd, gpu), dev(kd, gpu), dev(vd, gpu), scale))
                for j in range(len(batch)):
                    n = base[j] + s + 1
                    want = A.decode(qd[j], kv[j][0][:n], kv[j][1][:n], scale)
                    err = float(np.max(np.abs(od[j] - want)))
                    assert err <= TOL, f"request {i}.{j} decode step {s}: max abs error {err:.3e}"
        eng.release(b)
        st_ = eng.tree.stats()
        assert st_["locked_tokens"] == 0 and st_["free_slots"] + st_["cached_tokens"] <= n_pages
    assert reused > 0 and eng.tree.stats()["evicted_tokens"] > 0
