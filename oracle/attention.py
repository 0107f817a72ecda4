"""CPU oracle for attention over a prefix-shared KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU library (``prefix_shared_kv_amd``) and never imports it.

What is computed, and where the pages define it
-----------------------------------------------
"Prompt Caching" glossary (ultralytics), section "How prompt caching works":
prefill computes a key and a value per prompt token in every layer; during
decoding each new token attends to all of those keys and values; since
attention is causal, a token's K/V depend only on earlier tokens, so the K/V
of a shared prefix are identical across prompts and the cached copy can
replace recomputing it.  The worked GPT-2 example and the closing "related
terms" list state the consequence the method relies on: running only the new
tokens over the cached prefix gives the same next-token scores as a full
recompute, up to floating-point rounding.

So the method reaches exactly (up to rounding order) a result with a plain
definition, and this oracle is that definition: for every request, build the
logical K/V sequence (cached prefix, then the request's own new tokens, then
decoded tokens) and compute ordinary causal softmax attention for the
request's queries at their absolute positions.  It never looks at a KV pool
or an index table.

Precision: float64 throughout (the pages fix no precision).  Inputs are the
float32 arrays from the seeded generator (bf16-representable for bf16
workloads), upcast exactly.

Readings of points the pages leave open (each the plainest one consistent
with "same scores as a full recompute"):
  * causal alignment is by absolute position: new token i of a request whose
    cached prefix has P tokens sits at position P + i and sees keys 0..P+i,
    itself included;
  * softmax scale is an explicit argument (default 1/sqrt(head_dim));
  * grouped-query attention: q-head h reads kv-head floor(h * Hkv / Hq),
    i.e. contiguous groups of Hq/Hkv query heads per kv-head;
  * a decode step first stores the new token's K/V, then attends over the
    whole context including it.
"""
from __future__ import annotations

import numpy as np


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h (contiguous query-head groups)."""
    return (h * num_kv_heads) // num_q_heads


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float, last_key: np.ndarray) -> np.ndarray:
    """Softmax attention with a per-query visibility limit.

    q [n, D], k [L, D], v [L, D]; query i sees keys 0..last_key[i] inclusive.
    Two-pass softmax: subtract the row maximum, exponentiate, normalise.
    Returns [n, D] float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L = k.shape[0]
    s = sm_scale * (q @ k.T)
    hidden = np.arange(L)[None, :] > np.asarray(last_key)[:, None]
    s = np.where(hidden, -np.inf, s)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def extend(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, prefix_len: int, sm_scale: float) -> np.ndarray:
    """Attention outputs of one request's new tokens.

    q [E, Hq, D] are the queries of the E new tokens; k_ctx/v_ctx [P+E(+...), Hkv, D]
    hold the request's logical K/V sequence (cached prefix first).  New token i is at
    absolute position prefix_len + i.  Returns [E, Hq, D] float64.
    """
    E, Hq, D = q.shape
    Hkv = k_ctx.shape[1]
    out = np.empty((E, Hq, D), np.float64)
    last = prefix_len + np.arange(E)
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        out[:, h] = attend(q[:, h], k_ctx[:, g], v_ctx[:, g], sm_scale, last)
    return out


def decode(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, sm_scale: float) -> np.ndarray:
    """One decode query per head over the whole context k_ctx/v_ctx [L, Hkv, D]
    (the new token's own K/V is the last row).  q [Hq, D] -> [Hq, D] float64."""
    L = k_ctx.shape[0]
    return extend(q[None], k_ctx, v_ctx, L - 1, sm_scale)[0]


def kv_store(pool: np.ndarray, new: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """Pool after writing row i of ``new`` into slot slots[i] (a bit copy; every
    other slot unchanged).  Works on any dtype, e.g. uint16 bf16 bit patterns."""
    out = pool.copy()
    out[np.asarray(slots, np.int64)] = new
    return out

