"""GPU parity of the label distribution (rc_label_distribution) against the
float64 oracle: the chosen option bit-exact (decided on the same gathered
logits on both sides), probabilities within 2e-6, the expected index within
1e-4 and the confidence within 1e-5 (fp32 arithmetic of at most 64 terms)."""
import numpy as np
import pytest
import torch

from oracle import labels as L
from prefix_shared_kv_amd import api
from synth import workloads as W

pytestmark = pytest.mark.gpu

TOL_P, TOL_E, TOL_C = 2e-6, 1e-4, 1e-5


def run(gpu, logits_np, ids, counts=None, dtype=torch.float32, stride_pad=0, vocab=None):
    R, V = logits_np.shape
    buf = torch.zeros(R, V + stride_pad, dtype=dtype, device=gpu)
    buf[:, :V] = torch.from_numpy(logits_np).to(gpu).to(dtype)
    view = buf[:, :V]
    host_logits = view.float().cpu().numpy()  # the values the kernel reads (bf16-rounded when bf16)
    ids_d = torch.from_numpy(np.asarray(ids, np.int32)).to(gpu)
    cnt_d = None if counts is None else torch.from_numpy(np.asarray(counts, np.int32)).to(gpu)
    probs, ch, ex, cf = api.label_distribution(view, ids_d, cnt_d, vocab=vocab)
    torch.cuda.synchronize()
    return host_logits, probs.cpu().numpy(), ch.cpu().numpy(), ex.cpu().numpy(), cf.cpu().numpy()


def compare(host_logits, ids, counts, probs, ch, ex, cf, what):
    wp, wc, we, wf = L.classify(host_logits, list(ids), counts)
    assert np.array_equal(ch, wc), f"{what}: choice differs in rows {np.flatnonzero(ch != wc)[:8]}"
    assert np.max(np.abs(probs - wp)) <= TOL_P, f"{what}: probs {np.max(np.abs(probs - wp)):.2e}"
    assert np.max(np.abs(ex - we)) <= TOL_E, f"{what}: expected index {np.max(np.abs(ex - we)):.2e}"
    assert np.max(np.abs(cf - wf)) <= TOL_C, f"{what}: confidence {np.max(np.abs(cf - wf)):.2e}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows", [1, 5, 64, 257])
def test_full_vocabulary_rows(gpu, dtype, rows):
    logits = W.next_token_logits(1, rows)
    ids = W.label_token_ids(1)
    counts = W.option_counts(1, rows)
    counts[0] = 1
    if rows > 2:
        counts[1], counts[2] = 2, 64
    h, p, c, e, f = run(gpu, logits, ids, counts, dtype)
    compare(h, ids, counts, p, c, e, f, f"{dtype} rows={rows}")


def test_all_labels_without_counts_and_strided_rows(gpu):
    logits = W.next_token_logits(2, 33)
    ids = W.label_token_ids(2, 40)
    h, p, c, e, f = run(gpu, logits, ids, None, stride_pad=47)
    compare(h, ids, None, p, c, e, f, "strided")


def test_ties_go_to_the_lowest_option(gpu):
    g = np.random.default_rng(3)
    logits = W.next_token_logits(3, 16, vocab=1000)
    ids = np.arange(100, 164, dtype=np.int32)
    for r in range(16):  # several labels share the row's largest logit
        tied = g.choice(64, size=1 + r % 5, replace=False)
        logits[r, ids[tied]] = 50.0
    h, p, c, e, f = run(gpu, logits, ids)
    compare(h, ids, None, p, c, e, f, "ties")
    for r in range(16):
        assert c[r] == np.flatnonzero(h[r, ids] == 50.0)[0]


def test_huge_logits_stay_finite(gpu):
    logits = W.next_token_logits(4, 8, vocab=512) + np.float32(1e4)
    ids = np.arange(0, 512, 8, dtype=np.int32)
    h, p, c, e, f = run(gpu, logits, ids)
    assert np.all(np.isfinite(p)) and np.all(np.isfinite(f))
    compare(h, ids, None, p, c, e, f, "huge")


def test_point_mass_and_uniform(gpu):
    logits = np.zeros((2, 300), np.float32)
    logits[0, 17] = 200.0
    ids = np.arange(0, 64, dtype=np.int32)
    h, p, c, e, f = run(gpu, logits, ids)
    assert c[0] == 17 and p[0, 17] == 1.0 and f[0] == 1.0 and e[0] == 17.0
    assert np.allclose(p[1], 1 / 64, atol=1e-7) and abs(f[1]) < 1e-6 and abs(e[1] - 31.5) < 1e-4


def test_bad_label_ids_and_counts_are_flagged(gpu):
    err = torch.zeros(1, dtype=torch.int32, device=gpu)
    api.set_error_word(err)
    try:
        logits = W.next_token_logits(5, 4, vocab=200)
        ids = np.array([3, 250, 7, 9], np.int32)  # 250 is outside the vocabulary
        h, p, c, e, f = run(gpu, logits, ids, counts=[4, 0, 9, 2])
        assert int(err.item()) & 16
        assert np.all(p[:, 1] == 0)  # the bad label gets no probability
        # counts clamp into [1, 4]; the remaining labels renormalise among themselves
        good = [0, 2, 3]
        x = h[0, ids[good]].astype(np.float64)
        want = np.exp(x - x.max()) / np.exp(x - x.max()).sum()
        assert np.max(np.abs(p[0, good] - want)) <= TOL_P
        assert p[1, 0] == 1.0 and c[1] == 0  # count 0 -> one option
    finally:
        api.set_error_word(None)


def test_rejects_bad_arguments(gpu):
    logits = torch.zeros(2, 10, device=gpu)
    ids = torch.zeros(65, dtype=torch.int32, device=gpu)
    with pytest.raises(Exception):
        api.label_distribution(logits, ids)  # more than 64 labels
    with pytest.raises(Exception):
        api.label_distribution(logits, ids[:4], vocab=11)  # vocab beyond the row
