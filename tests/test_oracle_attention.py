"""Pins for the attention oracle: things other than the oracle itself that fix
what it must return (a library routine, scalar brute force, closed forms,
and the invariants the pages state)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _loops(q, k, v, sm_scale, last_key):
    """Scalar brute force: explicit loops over queries, keys and head dims."""
    n, D = len(q), len(q[0])
    out = []
    for i in range(n):
        scores = [sm_scale * sum(float(q[i][d]) * float(k[j][d]) for d in range(D)) for j in range(int(last_key[i]) + 1)]
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        tot = sum(w)
        out.append([sum(w[j] * float(v[j][d]) for j in range(len(w))) / tot for d in range(D)])
    return np.array(out)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attend_matches_scalar_loops(seed):
    q, k, v = _rand(seed, 5, 6), _rand(seed + 10, 9, 6), _rand(seed + 20, 9, 6)
    last = np.array([0, 3, 4, 8, 6])
    got = A.attend(q, k, v, 0.37, last)
    want = _loops(q, k, v, 0.37, last)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def _sdpa_bottom_right(q, k_ctx, v_ctx, P, scale):
    """torch SDPA (float64, CPU) with an explicit bottom-right causal mask and
    kv heads expanded to query heads in contiguous groups."""
    E, Hq, D = q.shape
    L, Hkv, _ = k_ctx.shape
    g = Hq // Hkv
    qt = torch.from_numpy(q).double().permute(1, 0, 2)  # [Hq, E, D]
    kt = torch.from_numpy(k_ctx).double().permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
    vt = torch.from_numpy(v_ctx).double().permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
    pos = P + torch.arange(E)[:, None]
    allowed = torch.arange(L)[None, :] <= pos
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv,P,E", [(4, 4, 0, 7), (4, 2, 5, 3), (8, 2, 17, 11), (6, 3, 30, 1)])
def test_extend_matches_torch_sdpa(Hq, Hkv, P, E):
    D = 16
    q = _rand(1, E, Hq, D)
    k = _rand(2, P + E, Hkv, D)
    v = _rand(3, P + E, Hkv, D)
    got = A.extend(q, k, v, P, 0.21)
    want = _sdpa_bottom_right(q, k, v, P, 0.21)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_decode_matches_torch_sdpa_over_whole_context():
    Hq, Hkv, D, L = 8, 2, 32, 50
    q, k, v = _rand(4, Hq, D), _rand(5, L, Hkv, D), _rand(6, L, Hkv, D)
    got = A.decode(q, k, v, 0.125)
    qt = torch.from_numpy(q).double()[:, None]  # [Hq, 1, D]
    kt = torch.from_numpy(k).double().permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0).contiguous()
    vt = torch.from_numpy(v).double().permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0).contiguous()
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.125)[:, 0].numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_single_key_gives_value_exactly():
    # the first token of a prefill sees only itself: softmax weight exactly 1
    q, k, v = _rand(7, 1, 4, 8), _rand(8, 1, 2, 8), _rand(9, 1, 2, 8)
    got = A.extend(q, k, v, 0, 0.5)
    for h in range(4):
        assert np.array_equal(got[0, h], v[0, h // 2])


def test_weights_sum_to_one():
    # V = 1 everywhere: every output is the sum of its softmax weights
    P, E, D = 37, 9, 16
    q, k = _rand(20, E, 4, D) * 3, _rand(21, P + E, 2, D) * 3
    got = A.extend(q, k, np.ones((P + E, 2, D)), P, 0.7)
    np.testing.assert_allclose(got, 1.0, rtol=0, atol=1e-14)
    got = A.decode(q[0], k, np.ones((P + E, 2, D)), 0.7)
    np.testing.assert_allclose(got, 1.0, rtol=0, atol=1e-14)


def test_zero_query_gives_causal_running_mean():
    P, E, D = 6, 5, 8
    k, v = _rand(10, P + E, 1, D), _rand(11, P + E, 1, D)
    q = np.zeros((E, 1, D))
    got = A.extend(q, k, v, P, 1.0)
    for i in range(E):
        np.testing.assert_allclose(got[i, 0], v[: P + i + 1, 0].mean(axis=0), rtol=0, atol=1e-14)


def test_equal_keys_give_running_mean_whatever_the_query():
    P, E, D = 4, 4, 8
    k = np.tile(_rand(12, 1, 1, D), (P + E, 1, 1)) * 3.0
    v = _rand(13, P + E, 1, D)
    q = _rand(14, E, 1, D) * 5.0
    got = A.extend(q, k, v, P, 1.0)
    for i in range(E):
        np.testing.assert_allclose(got[i, 0], v[: P + i + 1, 0].mean(axis=0), rtol=0, atol=1e-13)


def test_dominant_key_selects_its_value():
    L, D = 12, 8
    k, v = _rand(15, L, 1, D), _rand(16, L, 1, D)
    j = 7
    q = (k[j, 0] / np.linalg.norm(k[j, 0]) * 400.0)[None, None]
    k = k.copy()
    k[j, 0] *= 4.0  # make key j the clear argmax
    got = A.decode(q[0], k, v, 1.0)
    np.testing.assert_allclose(got[0], v[j, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("P", [1, 9, 24])
def test_cached_prefix_equals_full_recompute(P):
    # glossary worked example: only the new tokens run over the cached prefix and
    # give the scores a full recompute gives
    E, Hq, Hkv, D = 6, 4, 2, 16
    full_q = _rand(17, P + E, Hq, D)
    k, v = _rand(18, P + E, Hkv, D), _rand(19, P + E, Hkv, D)
    full = A.extend(full_q, k, v, 0, 0.3)
    cached = A.extend(full_q[P:], k, v, P, 0.3)
    np.testing.assert_allclose(cached, full[P:], rtol=0, atol=1e-13)


def test_any_split_point_gives_the_same_outputs():
    # "whatever radix split": recomputing part of the cached prefix changes nothing
    P, E, Hq, Hkv, D = 20, 5, 4, 4, 8
    q_all = _rand(20, P + E, Hq, D)
    k, v = _rand(21, P + E, Hkv, D), _rand(22, P + E, Hkv, D)
    ref = A.extend(q_all[P:], k, v, P, 0.4)
    for Pp in [0, 3, 11, 19]:
        got = A.extend(q_all[Pp:], k, v, Pp, 0.4)[P - Pp:]
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_gqa_equals_mha_on_repeated_kv():
    E, P, Hq, Hkv, D = 4, 7, 8, 2, 16
    q, k, v = _rand(23, E, Hq, D), _rand(24, P + E, Hkv, D), _rand(25, P + E, Hkv, D)
    got = A.extend(q, k, v, P, 0.25)
    k_rep = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1).numpy()
    v_rep = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1).numpy()
    want = A.extend(q, k_rep, v_rep, P, 0.25)
    np.testing.assert_array_equal(got, want)


def test_gqa_group_mapping_is_contiguous():
    assert [A.kv_head_of(h, 32, 8) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [A.kv_head_of(h, 12, 12) for h in range(3)] == [0, 1, 2]


def test_kv_store_is_a_bit_copy_into_slots():
    pool = np.arange(40, dtype=np.uint16).reshape(10, 2, 2)
    new = (np.arange(12, dtype=np.uint16) + 1000).reshape(3, 2, 2)
    slots = np.array([7, 0, 4], np.int32)
    out = A.kv_store(pool, new, slots)
    for i, s in enumerate(slots):
        assert np.array_equal(out[s], new[i])
    for s in set(range(10)) - set(slots.tolist()):
        assert np.array_equal(out[s], pool[s])
    assert np.array_equal(pool, np.arange(40, dtype=np.uint16).reshape(10, 2, 2))  # input untouched
