"""Seeded synthetic workloads for attention over a prefix-shared KV pool.

This module only *draws inputs*: token ids, keys, values and queries, the
shape of the prefix tree that requests share, and the order in which pool
slots are handed out.  It contains none of the arithmetic of the method
(no attention, no matching, no slot bookkeeping), so both the GPU path and
the CPU oracle can consume its outputs without sharing any logic.

Workload shapes follow the use cases the pages name:
  * "Prompt Caching" glossary (ultralytics), worked GPT-2 example: a 409-token
    system prompt prefilled once, then two questions of 8 and 7 tokens that
    run alone over the cached prefix (config ``gpt2_system_prompt``);
  * same page, list of workloads with long shared prefixes (few-shot prompts,
    chat history) and the SGLang summary (unite.ai), RadixAttention section:
    few-shot batches and multi-turn chat trees (configs ``few_shot`` and
    ``multi_turn_tree``);
  * openjev-sglang tutorial (aiezz), "how inference works": one warmed shared
    prefix plus many single-token branches (config ``classify64``), and heavy
    decode over contexts shared by groups of requests (``heavy_decode``).

Design of the draws
-------------------
* K/V are keyed by (tree node, offset): every request whose context contains a
  node sees bit-identical K/V for it.  This is the causal-reuse property the
  glossary states (a token's K/V depend only on the tokens before it), built in
  by construction.
* Q is keyed by (request, position).
* Values are N(0, std) in float32, then rounded to bfloat16 (round to nearest
  even) for bf16 workloads; arrays are returned as float32 holding exactly the
  representable values, so upcasting on either side is exact.
* Token ids are uniform in [0, 50257); the first tokens of all children of a
  node are forced distinct, so the longest cached prefix of a request is
  exactly its tree path.
* Streams are ``SeedSequence(seed, spawn_key=(TAG, id...))`` so any part can be
  regenerated alone (the oracle recomputes only what it samples).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

VOCAB = 50257

# stream tags (arbitrary distinct integers)
_T_NODE_TOK, _T_NODE_K, _T_NODE_V = 11, 12, 13
_T_NODE_DEV = 14
_T_EXT_TOK, _T_EXT_Q, _T_EXT_K, _T_EXT_V = 21, 22, 23, 24
_T_DEC_Q, _T_DEC_K, _T_DEC_V = 31, 32, 33
_T_PRE_Q = 41
_T_SLOTS, _T_LEN, _T_FIRST = 51, 52, 53
_T_PFX_K, _T_PFX_V, _T_PFX_Q = 61, 62, 63
_T_LOGITS, _T_LABELS, _T_OPTIONS = 71, 72, 73


def rng(seed: int, tag: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tag,) + tuple(int(i) for i in ids))))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even); float32 out.
    On the bit pattern: add 0x7FFF plus the lowest kept bit, then clear the low 16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def prefix_hashes(tokens: np.ndarray) -> np.ndarray:
    """h[p] identifies tokens[:p+1] (a polynomial hash modulo the prime 2^61 - 1)."""
    M, h, out = (1 << 61) - 1, 0, np.zeros(len(tokens), np.int64)
    for p, t in enumerate(np.asarray(tokens, np.int64).tolist()):
        h = (h * 1000003 + t + 1) % M
        out[p] = h
    return out


def prefix_keyed_kv(seed: int, tokens: np.ndarray, shape: "Shape", start: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """K and V [len(tokens) - start, Hkv, D] for positions start.. of a sequence.  Position p's
    values come from a stream keyed by tokens[:p+1] alone, so every sequence with the same first
    p+1 tokens gets bit-identical K/V at p, whatever was cached, evicted or recomputed."""
    h = prefix_hashes(tokens)
    n = len(tokens) - start
    k = np.zeros((n, shape.num_kv_heads, shape.head_dim), np.float32)
    v = np.zeros_like(k)
    for i in range(n):
        key = (int(h[start + i]) & 0xFFFFFFFF, int(h[start + i]) >> 32)
        k[i] = rng(seed, _T_PFX_K, *key).standard_normal(k.shape[1:], dtype=np.float32) * shape.std
        v[i] = rng(seed, _T_PFX_V, *key).standard_normal(k.shape[1:], dtype=np.float32) * shape.std
    if shape.dtype == "bf16":
        k, v = round_bf16(k), round_bf16(v)
    return k, v


def keyed_q(seed: int, shape: "Shape", n: int, *ids: int) -> np.ndarray:
    """Queries [n, Hq, D] from a stream keyed by ids."""
    q = rng(seed, _T_PFX_Q, *ids).standard_normal((n, shape.num_q_heads, shape.head_dim), dtype=np.float32)
    q *= shape.std
    return round_bf16(q) if shape.dtype == "bf16" else q


def label_token_ids(seed: int, n: int = 64, vocab: int = VOCAB) -> np.ndarray:
    """n distinct token ids standing for the answer labels A..Z, AA, AB, ... (int32)."""
    return rng(seed, _T_LABELS).choice(vocab, size=n, replace=False).astype(np.int32)


def next_token_logits(seed: int, rows: int, vocab: int = VOCAB, std: float = 3.0, row: int = 0) -> np.ndarray:
    """Next-token logits [rows, vocab] float32, N(0, std): the rows of one batch of branches."""
    return rng(seed, _T_LOGITS, row).standard_normal((rows, vocab), dtype=np.float32) * np.float32(std)


def option_counts(seed: int, rows: int, lo: int = 2, hi: int = 64) -> np.ndarray:
    """Options per question, uniform in [lo, hi] (int32)."""
    return rng(seed, _T_OPTIONS).integers(lo, hi + 1, size=rows).astype(np.int32)


@dataclasses.dataclass
class Shape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    std: float = 1.0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclasses.dataclass
class Node:
    id: int
    parent: int  # -1 for children of the (empty) root
    tokens: np.ndarray  # int32


@dataclasses.dataclass
class Request:
    id: int
    path: List[int]  # node ids, root side first
    ext_tokens: np.ndarray  # int32, the request's own new tokens
    n_decode: int


class Workload:
    """A tree of cached segments plus a batch of requests hanging off it."""

    def __init__(self, name: str, shape: Shape, seed: int, nodes: List[Node], requests: List[Request],
                 prefill_nodes: Sequence[int] = (), shuffle_slots: bool = False, extra_slots: int = 0):
        self.name = name
        self.shape = shape
        self.seed = seed
        self.nodes = nodes
        self.requests = requests
        self.prefill_nodes = list(prefill_nodes)
        self.sm_scale = 1.0 / float(np.sqrt(shape.head_dim))
        n_cached = sum(len(n.tokens) for n in nodes)
        n_new = sum(len(r.ext_tokens) + r.n_decode for r in requests)
        self.pool_slots = int(n_cached + n_new + extra_slots)
        self.shuffle_slots = shuffle_slots

    # ---- structure -------------------------------------------------------
    def node_start(self, nid: int) -> int:
        """Absolute position of the node's first token (tokens on the path before it)."""
        s, p = 0, self.nodes[nid].parent
        while p >= 0:
            s += len(self.nodes[p].tokens)
            p = self.nodes[p].parent
        return s

    def prefix_tokens(self, r: Request) -> np.ndarray:
        if not r.path:
            return np.zeros(0, np.int32)
        return np.concatenate([self.nodes[n].tokens for n in r.path]).astype(np.int32)

    def prompt_tokens(self, r: Request) -> np.ndarray:
        return np.concatenate([self.prefix_tokens(r), r.ext_tokens]).astype(np.int32)

    def free_order(self) -> Optional[np.ndarray]:
        """Initial free-slot order for the pool: identity, or a seeded permutation."""
        if not self.shuffle_slots:
            return None
        return rng(self.seed, _T_SLOTS).permutation(self.pool_slots).astype(np.int32)

    # ---- values ----------------------------------------------------------
    def _vals(self, shape, tag, *ids) -> np.ndarray:
        x = rng(self.seed, tag, *ids).standard_normal(shape, dtype=np.float32)
        if self.shape.std != 1.0:
            x = (x * np.float32(self.shape.std)).astype(np.float32)
        return round_bf16(x) if self.shape.dtype == "bf16" else x

    def node_kv(self, nid: int) -> Tuple[np.ndarray, np.ndarray]:
        n = len(self.nodes[nid].tokens)
        s = (n, self.shape.num_kv_heads, self.shape.head_dim)
        return self._vals(s, _T_NODE_K, nid), self._vals(s, _T_NODE_V, nid)

    def node_kv_device(self, nid: int, device):
        """Node K/V drawn on a GPU by torch's seeded generator: [n, Hkv, D] tensors
        in the workload dtype.  For pools too large to draw on the host (the
        heavy-decode workload holds 9 GB); repeated calls give the same bits, so
        the oracle side regenerates the nodes it samples and copies them out."""
        import torch
        seed = int(np.random.SeedSequence(self.seed, spawn_key=(_T_NODE_DEV, int(nid))).generate_state(1, np.uint64)[0] >> 1)
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        n = len(self.nodes[nid].tokens)
        s = (n, self.shape.num_kv_heads, self.shape.head_dim)
        dt = torch.bfloat16 if self.shape.dtype == "bf16" else torch.float32
        k = torch.randn(s, generator=g, device=device, dtype=torch.float32)
        v = torch.randn(s, generator=g, device=device, dtype=torch.float32)
        if self.shape.std != 1.0:
            k, v = k * self.shape.std, v * self.shape.std
        return k.to(dt), v.to(dt)

    def node_prefill_q(self, nid: int) -> np.ndarray:
        """Queries for prefilling a node's own tokens (extend with the node as new tokens)."""
        n = len(self.nodes[nid].tokens)
        return self._vals((n, self.shape.num_q_heads, self.shape.head_dim), _T_PRE_Q, nid)

    def ext_qkv(self, rid: int):
        e = len(self.requests[rid].ext_tokens)
        sh = self.shape
        return (self._vals((e, sh.num_q_heads, sh.head_dim), _T_EXT_Q, rid),
                self._vals((e, sh.num_kv_heads, sh.head_dim), _T_EXT_K, rid),
                self._vals((e, sh.num_kv_heads, sh.head_dim), _T_EXT_V, rid))

    def dec_qkv(self, rid: int, t: int):
        sh = self.shape
        return (self._vals((sh.num_q_heads, sh.head_dim), _T_DEC_Q, rid, t),
                self._vals((sh.num_kv_heads, sh.head_dim), _T_DEC_K, rid, t),
                self._vals((sh.num_kv_heads, sh.head_dim), _T_DEC_V, rid, t))

    def prefix_kv(self, r: Request) -> Tuple[np.ndarray, np.ndarray]:
        sh = self.shape
        if not r.path:
            z = np.zeros((0, sh.num_kv_heads, sh.head_dim), np.float32)
            return z, z.copy()
        ks, vs = zip(*(self.node_kv(n) for n in r.path))
        return np.concatenate(ks), np.concatenate(vs)

    def context_kv(self, rid: int, n_decoded: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Logical K/V sequence of a request: path nodes, own new tokens, first n_decoded decode tokens."""
        r = self.requests[rid]
        pk, pv = self.prefix_kv(r)
        _, ek, ev = self.ext_qkv(rid)
        parts_k, parts_v = [pk, ek], [pv, ev]
        for t in range(n_decoded):
            _, dk, dv = self.dec_qkv(rid, t)
            parts_k.append(dk[None])
            parts_v.append(dv[None])
        return np.concatenate(parts_k), np.concatenate(parts_v)


# ---- tree construction helpers --------------------------------------------

class _TreeBuilder:
    def __init__(self, seed: int):
        self.seed = seed
        self.nodes: List[Node] = []
        self.children: dict = {}  # parent id -> list of (kind, id)

    def _first_tokens(self, parent: int, count: int) -> np.ndarray:
        g = rng(self.seed, _T_FIRST, parent + 1)
        return g.choice(VOCAB, size=count, replace=False).astype(np.int32)

    def add_children(self, parent: int, lengths: Sequence[int]) -> List[int]:
        firsts = self._first_tokens(parent, len(lengths))
        ids = []
        for i, n in enumerate(lengths):
            nid = len(self.nodes)
            toks = rng(self.seed, _T_NODE_TOK, nid).integers(0, VOCAB, size=n, dtype=np.int64).astype(np.int32)
            toks[0] = firsts[i]
            self.nodes.append(Node(nid, parent, toks))
            ids.append(nid)
        return ids

    def path(self, nid: int) -> List[int]:
        p = []
        while nid >= 0:
            p.append(nid)
            nid = self.nodes[nid].parent
        return p[::-1]


def _ext_tokens(seed: int, leaf_of_req: Sequence[int], lengths: Sequence[int]) -> List[np.ndarray]:
    """New tokens of each request; first tokens distinct among requests under the same node."""
    out = [None] * len(lengths)
    by_parent: dict = {}
    for rid, p in enumerate(leaf_of_req):
        by_parent.setdefault(p, []).append(rid)
    for p, rids in by_parent.items():
        # distinct from each other; offset the stream so they also differ from node children draws
        firsts = rng(seed, _T_FIRST, 10_000_000 + p + 1).choice(VOCAB, size=len(rids), replace=False)
        for i, rid in enumerate(rids):
            t = rng(seed, _T_EXT_TOK, rid).integers(0, VOCAB, size=lengths[rid], dtype=np.int64).astype(np.int32)
            if lengths[rid] > 0:
                t[0] = firsts[i]
            out[rid] = t
    return out


def _make_requests(tb: _TreeBuilder, leaf_of_req: Sequence[int], ext_lens: Sequence[int], n_decode: int) -> List[Request]:
    exts = _ext_tokens(tb.seed, leaf_of_req, ext_lens)
    return [Request(i, tb.path(p) if p >= 0 else [], exts[i], n_decode) for i, p in enumerate(leaf_of_req)]


def _fix_ext_vs_children(tb: _TreeBuilder, reqs: List[Request]):
    """Make a request's first new token differ from every child node's first token of its leaf."""
    kids: dict = {}
    for n in tb.nodes:
        kids.setdefault(n.parent, set()).add(int(n.tokens[0]))
    for r in reqs:
        leaf = r.path[-1] if r.path else -1
        used = kids.get(leaf, set())
        if len(r.ext_tokens) and int(r.ext_tokens[0]) in used:
            v = int(r.ext_tokens[0])
            while v in used:
                v = (v + 1) % VOCAB
            r.ext_tokens[0] = v


# ---- the five workloads -----------------------------------------------------

def tiny_fp32(seed: int = 1) -> Workload:
    """fp32, 4 q-heads = 4 kv-heads, head_dim 64, pool of 512 slots; 2 requests
    share a 128-token prefix and extend by 8 each; 4 decode steps."""
    tb = _TreeBuilder(seed)
    (pre,) = tb.add_children(-1, [128])
    reqs = _make_requests(tb, [pre, pre], [8, 8], 4)
    _fix_ext_vs_children(tb, reqs)
    w = Workload("tiny_fp32", Shape(4, 4, 64, "f32"), seed, tb.nodes, reqs, prefill_nodes=[pre])
    w.pool_slots = 512
    return w


def gpt2_system_prompt(seed: int = 2) -> Workload:
    """GPT-2-small-shaped layer, bf16, 12 heads, head_dim 64: a 409-token system
    prompt prefilled once, two branches of 8 and 7 new tokens, 32 decode steps
    each; q, k, v ~ N(0,1) scaled by 1/sqrt(64)."""
    tb = _TreeBuilder(seed)
    (pre,) = tb.add_children(-1, [409])
    reqs = _make_requests(tb, [pre, pre], [8, 7], 32)
    _fix_ext_vs_children(tb, reqs)
    return Workload("gpt2_system_prompt", Shape(12, 12, 64, "bf16", std=0.125), seed, tb.nodes, reqs,
                    prefill_nodes=[pre])


def few_shot(seed: int = 3, n_req: int = 64, prefix: int = 2048, ext: int = 64, n_decode: int = 128) -> Workload:
    """Llama-3-8B-shaped GQA layer (32/8 heads, head_dim 128), bf16: 64 requests
    share a 2048-token few-shot prefix, extend by 64 tokens, decode 128 steps."""
    tb = _TreeBuilder(seed)
    (pre,) = tb.add_children(-1, [prefix])
    reqs = _make_requests(tb, [pre] * n_req, [ext] * n_req, n_decode)
    _fix_ext_vs_children(tb, reqs)
    return Workload("few_shot", Shape(32, 8, 128, "bf16"), seed, tb.nodes, reqs, prefill_nodes=[pre])


def multi_turn_tree(seed: int = 4, depth: int = 4, fanout: int = 4, seg_lo: int = 256, seg_hi: int = 1024,
                    ext: int = 128, n_decode: int = 256, shuffle: bool = True) -> Workload:
    """Multi-turn chat radix tree, GQA 32/8, head_dim 128, bf16: depth 4,
    branching 4 (256 leaves), segment lengths uniform in [256, 1024]; each leaf
    request extends by 128 tokens, then decodes 256 steps; pool slots handed out
    in a seeded random order."""
    tb = _TreeBuilder(seed)
    level = [-1]
    for _ in range(depth):
        nxt = []
        for p in level:
            lens = rng(seed, _T_LEN, p + 1).integers(seg_lo, seg_hi + 1, size=fanout)
            nxt += tb.add_children(p, [int(x) for x in lens])
        level = nxt
    reqs = _make_requests(tb, level, [ext] * len(level), n_decode)
    _fix_ext_vs_children(tb, reqs)
    return Workload("multi_turn_tree", Shape(32, 8, 128, "bf16"), seed, tb.nodes, reqs, shuffle_slots=shuffle)


def classify64(seed: int = 5, prefix: int = 4096, n_branch: int = 64, lo: int = 2, hi: int = 16) -> Workload:
    """64-way single-token classification: GQA 32/4, head_dim 128, bf16; a
    4096-token shared prefix prefilled once, 64 branches of 2..16 label tokens
    (one extend pass)."""
    tb = _TreeBuilder(seed)
    (pre,) = tb.add_children(-1, [prefix])
    lens = [int(x) for x in rng(seed, _T_LEN, 0).integers(lo, hi + 1, size=n_branch)]
    reqs = _make_requests(tb, [pre] * n_branch, lens, 0)
    _fix_ext_vs_children(tb, reqs)
    return Workload("classify64", Shape(32, 4, 128, "bf16"), seed, tb.nodes, reqs, prefill_nodes=[pre])


def heavy_decode(seed: int = 6, groups: int = 64, per_group: int = 16, shared: int = 4096, unique: int = 4096,
                 n_decode: int = 8) -> Workload:
    """Heavy decode: GQA 32/4, head_dim 128, bf16; 1024 requests over 8192-token
    contexts, 4096 shared within each group of 16 plus 4096 unique, all cached;
    8 decode steps (step t attends over 8192 + t keys)."""
    tb = _TreeBuilder(seed)
    gnodes = tb.add_children(-1, [shared] * groups)
    leaves = []
    for g in gnodes:
        leaves += tb.add_children(g, [unique] * per_group)
    reqs = _make_requests(tb, leaves, [0] * len(leaves), n_decode)
    return Workload("heavy_decode", Shape(32, 4, 128, "bf16"), seed, tb.nodes, reqs)


CONFIGS = {
    "tiny_fp32": tiny_fp32,
    "gpt2_system_prompt": gpt2_system_prompt,
    "few_shot": few_shot,
    "multi_turn_tree": multi_turn_tree,
    "classify64": classify64,
    "heavy_decode": heavy_decode,
}
