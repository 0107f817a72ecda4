"""Label-restricted next-token distribution for single-token classification.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with ``prefix_shared_kv_amd`` and never imports it.

What the pages fix (openjev-sglang tutorial, aiezz):
  * "how inference works", step 5: only the log-probabilities of the allowed
    answer labels are taken, and they are renormalised with a stable softmax;
  * the question types: Choice returns the most probable option and the whole
    distribution; Bool the normalised probability of "yes"; Score the expected
    zero-based level, each level's index weighted by its probability;
  * labels run A..Z, then checked single-token pairs (AA, AB, ...), 64 at most;
  * "interpret confidence carefully": confidence = 1 - H(p) / log(n) for n
    options, between 0 and 1; equal probabilities give 0 and a point mass 1.

Readings where the pages are silent:
  * a question with k options uses the first k labels of the label list, so
    the label of option i is label i (the distribution is over options in
    label order);
  * the most probable option is decided on the gathered logits (the softmax is
    monotone), ties going to the lowest index;
  * H uses the natural logarithm with 0 log 0 = 0 (the base cancels in the
    ratio); a question with one option has confidence 1 (a point mass);
  * Bool is the two-option case with the labels ordered (yes, no): its answer
    is p[0].
Everything is float64.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


def distribution(logits_row: np.ndarray, label_ids: Sequence[int]) -> np.ndarray:
    """Stable softmax over the logits of the given label tokens."""
    x = np.asarray(logits_row, np.float64)[np.asarray(label_ids, np.int64)]
    e = np.exp(x - x.max())
    return e / e.sum()


def choice(logits_row: np.ndarray, label_ids: Sequence[int]) -> int:
    x = np.asarray(logits_row, np.float64)[np.asarray(label_ids, np.int64)]
    return int(np.flatnonzero(x == x.max())[0])


def expected_index(p: np.ndarray) -> float:
    return float(sum(i * pi for i, pi in enumerate(p)))


def confidence(p: np.ndarray) -> float:
    n = len(p)
    if n == 1:
        return 1.0
    h = -sum(pi * math.log(pi) for pi in p if pi > 0)
    return 1.0 - h / math.log(n)


def classify(logits: np.ndarray, label_ids: Sequence[int],
             counts: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Per row r with counts[r] options (default: all labels): probabilities [rows, n_labels]
    (zero past the row's options), choice, expected index and confidence."""
    logits = np.asarray(logits)
    R, L = logits.shape[0], len(label_ids)
    counts = [L] * R if counts is None else list(counts)
    probs = np.zeros((R, L))
    ch = np.zeros(R, np.int64)
    ex = np.zeros(R)
    cf = np.zeros(R)
    for r in range(R):
        ids = list(label_ids)[:counts[r]]
        p = distribution(logits[r], ids)
        probs[r, :len(p)] = p
        ch[r] = choice(logits[r], ids)
        ex[r] = expected_index(p)
        cf[r] = confidence(p)
    return probs, ch, ex, cf
