"""The seeded generators: determinism, shapes and the structural promises the
workloads rely on (distinct sibling first tokens, bf16-representable values)."""
import numpy as np

from synth import workloads as W


def test_same_seed_same_bits():
    a, b = W.few_shot(n_req=4, prefix=64, ext=8, n_decode=2), W.few_shot(n_req=4, prefix=64, ext=8, n_decode=2)
    assert np.array_equal(a.nodes[0].tokens, b.nodes[0].tokens)
    for x, y in zip(a.node_kv(0), b.node_kv(0)):
        assert np.array_equal(x, y)
    for x, y in zip(a.ext_qkv(3), b.ext_qkv(3)):
        assert np.array_equal(x, y)


def test_bf16_values_are_representable():
    w = W.gpt2_system_prompt()
    k, v = w.node_kv(0)
    bits = k.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    assert abs(float(k.std()) - 0.125) < 0.01


def test_sibling_first_tokens_distinct_and_paths():
    w = W.multi_turn_tree(seg_lo=4, seg_hi=8, ext=3, n_decode=1)
    assert len(w.nodes) == 4 + 16 + 64 + 256
    assert len(w.requests) == 256
    kids = {}
    for n in w.nodes:
        kids.setdefault(n.parent, []).append(int(n.tokens[0]))
    for firsts in kids.values():
        assert len(set(firsts)) == len(firsts)
    for r in w.requests:
        assert len(r.path) == 4
        used = set(int(w.nodes[c].tokens[0]) for c in range(len(w.nodes)) if w.nodes[c].parent == r.path[-1])
        assert int(r.ext_tokens[0]) not in used
    perm = w.free_order()
    assert sorted(perm.tolist()) == list(range(w.pool_slots))


def test_context_kv_is_node_keyed():
    w = W.few_shot(n_req=3, prefix=16, ext=4, n_decode=2)
    k0, _ = w.context_kv(0, 2)
    k1, _ = w.context_kv(1, 2)
    assert k0.shape == (16 + 4 + 2, 8, 128)
    assert np.array_equal(k0[:16], k1[:16])
    assert not np.array_equal(k0[16:], k1[16:])


def test_round_bf16_matches_torch_conversion():
    # random values over many binades, exact ties (low half 0x8000) with even and odd kept bits,
    # values one ulp either side of a tie, subnormals, zeros
    import torch
    g = np.random.default_rng(7)
    x = (g.standard_normal(200000) * np.exp2(g.integers(-130, 120, 200000))).astype(np.float32)
    hi = g.integers(0, 1 << 16, 20000, dtype=np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001]).astype(np.uint32)
    ties = ties[np.isfinite(ties.view(np.float32))].view(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-45, -3e-39, 1.0, 65504.0])])
    x = x[np.isfinite(x) & (np.abs(x) < 3.3e38)]
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(W.round_bf16(x).view(np.uint32), want.view(np.uint32))
