"""Feed a seeded Workload through the GPU path (prefix_shared_kv_amd.engine).

Glue for tests and the benchmark: it uploads generator outputs and calls the
engine in serving order.  It computes nothing itself and never touches the
CPU oracle; callers compare what it returns with the oracle separately.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from prefix_shared_kv_amd.api import KVShape
from prefix_shared_kv_amd.engine import Batch, DecodeState, Engine

from .workloads import Workload

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def up(x: np.ndarray, w: Workload, device) -> torch.Tensor:
    """Host float32 array (bf16-representable for bf16 workloads) -> device tensor of the workload dtype."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device).to(TORCH_DT[w.shape.dtype])


def kv_shape(w: Workload, pool_slots: Optional[int] = None) -> KVShape:
    s = w.shape
    return KVShape(s.num_q_heads, s.num_kv_heads, s.head_dim, TORCH_DT[s.dtype], pool_slots or w.pool_slots)


def make_engine(w: Workload, device="cuda", stride: Optional[int] = None, max_rows: Optional[int] = None,
                pool_slots: Optional[int] = None) -> Engine:
    longest = max(len(w.prompt_tokens(r)) + r.n_decode + 1 for r in w.requests)
    longest = max([longest] + [w.node_start(n) + len(w.nodes[n].tokens) + 1 for n in range(len(w.nodes))])
    stride = stride or longest
    rows = max_rows or (len(w.requests) + len(w.prefill_nodes) + 1)
    return Engine(kv_shape(w, pool_slots), stride, rows, device, free_order=w.free_order())


def node_order(w: Workload) -> List[int]:
    """Nodes with parents before children."""
    depth = {}
    for n in w.nodes:
        d, p = 0, n.parent
        while p >= 0:
            d, p = d + 1, w.nodes[p].parent
        depth[n.id] = d
    return sorted(range(len(w.nodes)), key=lambda i: (depth[i], i))


def path_tokens(w: Workload, nid: int) -> np.ndarray:
    path = []
    while nid >= 0:
        path.append(nid)
        nid = w.nodes[nid].parent
    return np.concatenate([w.nodes[i].tokens for i in reversed(path)]).astype(np.int32)


def populate(eng: Engine, w: Workload, node_ids: Optional[Sequence[int]] = None, device="cuda",
             device_values: bool = False) -> None:
    """Put cached nodes' K/V into the pool and the tree (as if computed earlier).
    device_values: draw them with Workload.node_kv_device instead of on the host."""
    ids = node_order(w) if node_ids is None else list(node_ids)
    for nid in ids:
        if device_values:
            k, v = w.node_kv_device(nid, device)
        else:
            k, v = (up(x, w, device) for x in w.node_kv(nid))
        eng.populate(path_tokens(w, nid), k, v, expect_cached=w.node_start(nid))


def prefill_nodes(eng: Engine, w: Workload, device="cuda") -> Dict[int, torch.Tensor]:
    """Prefill each prefill node as an extend with an empty prefix, then cache it."""
    out = {}
    for nid in w.prefill_nodes:
        toks = path_tokens(w, nid)
        b = eng.schedule([toks])
        start = w.node_start(nid)
        if int(b.prefix_lens[0]) != start or int(b.extend_lens[0]) != len(w.nodes[nid].tokens):
            raise RuntimeError(f"prefill of node {nid}: matched {b.prefix_lens[0]}, expected {start}")
        k, v = w.node_kv(nid)
        q = w.node_prefill_q(nid)
        out[nid] = eng.extend(b, up(q, w, device), up(k, w, device), up(v, w, device), w.sm_scale)
        eng.commit(b)
        eng.release(b)
    return out


def extend_requests(eng: Engine, w: Workload, rids: Optional[Sequence[int]] = None, device="cuda", commit=True,
                    cascade=False):
    """Schedule requests (prompt = path + own tokens, decode slots reserved) and run the extend
    (cascade: from the shared-prefix plan).  Returns (batch, o) with o [sum E, Hq, D] in request order."""
    rids = list(range(len(w.requests))) if rids is None else list(rids)
    reqs = [w.requests[i] for i in rids]
    reserve = max(r.n_decode for r in reqs) if reqs else 0
    b = eng.schedule([w.prompt_tokens(r) for r in reqs], reserve=reserve)
    expect = [len(w.prefix_tokens(r)) for r in reqs]
    if b.prefix_lens.tolist() != expect:
        raise RuntimeError(f"matched prefixes {b.prefix_lens.tolist()[:8]}.. differ from the workload's {expect[:8]}..")
    qs, ks, vs = zip(*(w.ext_qkv(i) for i in rids))
    q, k, v = (up(np.concatenate(x), w, device) for x in (qs, ks, vs))
    o = eng.extend(b, q, k, v, w.sm_scale, cascade=cascade)
    if commit:
        eng.commit(b)
    return b, o


def schedule_decode_only(eng: Engine, w: Workload, rids: Optional[Sequence[int]] = None) -> Batch:
    """Requests whose whole prompt is cached: schedule the first decode token as the one
    uncached token, with slots reserved for the remaining steps."""
    rids = list(range(len(w.requests))) if rids is None else list(rids)
    reqs = [w.requests[i] for i in rids]
    n = max(r.n_decode for r in reqs)
    toks = [np.concatenate([w.prompt_tokens(r), np.array([0], np.int32)]) for r in reqs]
    b = eng.schedule(toks, reserve=n - 1)
    if b.extend_lens.tolist() != [1] * len(reqs):
        raise RuntimeError("decode-only requests must have their whole prompt cached")
    return b


def decode_inputs(w: Workload, rids: Sequence[int], t: int, device="cuda"):
    qs, ks, vs = zip(*(w.dec_qkv(i, t) for i in rids))
    return tuple(up(np.stack(x), w, device) for x in (qs, ks, vs))
