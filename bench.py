"""Benchmark: one step = the whole hot path over one batch of a seeded
synthetic workload on one MI355X.  Prints one JSON line.

Default workload (--workload classify_heavy): 64-way single-token
classification plus heavy decode; GQA 32 q-heads / 4 kv-heads, head_dim 128,
bf16.
  * classification: a fresh 4096-token document is prefilled (an extend over an
    empty prefix) and cached, then 64 label branches of 2..16 tokens extend over
    it in one pass;
  * heavy decode: 1024 requests over 8192-token cached contexts (64 groups of 16
    share 4096 tokens, each request owns 4096 more), 8 decode steps.
The pool holds the 4.46M cached positions (9.1 GB of K and V).

A step, all of it inside the timed region:
  schedule the document (radix match, slots, table rows: host C++) -> upload
  its K/V scatter and prefill extend (HIP, MFMA); commit
  schedule the 64 branches; their scatter; their extend over a shared-prefix
  plan (host C++ planner, then the split-K kernel and merge: the document is
  read once per 16 label tokens, not once per branch); commit
  schedule the 1024 decode requests (their 8192 tokens are cached)
  decode share plan from the tree (host C++) -> upload
  8 decode steps: decode, which also stores the step's K/V, then merge (HIP)
  release of the decode slots
Tokens per step: 4096 + the branches' label tokens + 1024 x 8.

--workload multi_turn_tree: GQA 32/8; a cached radix tree of depth 4 and
branching 4 (340 segments of U[256,1024] tokens, 256 leaves), pool slots
handed out in a seeded random order; each leaf request brings 128 new tokens
(scatter, extend, commit), then decodes 256 tokens.

Inputs (q, k, v and the token batches) are made before timing; q, k and v
are drawn on the GPU and stay resident in HBM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
ROOT = os.path.dirname(os.path.abspath(__file__))
# the decode kernel's sources: a traffic figure stands only while these are unchanged
# what the decode kernel's code depends on: its sources and the build flags
KERNEL_SOURCES = [os.path.join(ROOT, "prefix_shared_kv_amd", "csrc", f)
                  for f in ("decode.hip", "attn_tile.h", "hip_common.h")] + [
                  os.path.join(ROOT, "prefix_shared_kv_amd", "build.py")]
METRIC = "extend-attn TFLOP/s (% MFMA peak) + decode-attn HBM GB/s, tokens/s, 1 GPU"


def traffic_file(workload: str) -> str:
    """HBM bytes per launch of the decode kernel from rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters, with the sha256 of the kernel source they were taken on."""
    return os.path.join(ROOT, "profiles", f"decode_attention_{workload}_traffic.txt")


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """Counter-measured bytes per decode launch, or None when absent or taken
    on a different kernel source."""
    try:
        kv = {}
        for line in open(traffic_file(workload)):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel_sources_sha256") != kernel_sources_sha256():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration():
    """kv_store of 65536 rows (K and V, 8 x 128 bf16 each) into slots 0..65535:
    reads 2 x 128 MiB + the slot list, writes 2 x 128 MiB."""
    import torch

    import prefix_shared_kv_amd as pk
    dev = torch.device("cuda:0")
    n, h, d = 65536, 8, 128
    kvs = pk.KVShape(32, h, d, torch.bfloat16, n)
    k_pool = torch.zeros((n, h, d), dtype=torch.bfloat16, device=dev)
    v_pool = torch.zeros_like(k_pool)
    k = torch.randn((n, h, d), device=dev).to(torch.bfloat16)
    v = torch.randn((n, h, d), device=dev).to(torch.bfloat16)
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    for _ in range(5):
        pk.kv_store(kvs, k_pool, v_pool, k, v, slots)
    torch.cuda.synchronize()
    if not (torch.equal(k_pool, k) and torch.equal(v_pool, v)):
        raise RuntimeError("calibration copy mismatch")
    row = h * d * 2
    print(json.dumps({"calibration": "kv_store into contiguous slots", "launches": 5,
                      "read_bytes_per_launch": 2 * n * row + 4 * n, "write_bytes_per_launch": 2 * n * row}))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=["classify_heavy", "multi_turn_tree"], default="classify_heavy")
    ap.add_argument("--chunk", type=int, default=None,
                    help="decode split size, nominal positions per work item (default: 4096 for classify_heavy, "
                         "1024 for multi_turn_tree)")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="decode steps per step (default 8 for classify_heavy, 256 for multi_turn_tree)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=16, help="requests in the oracle's decode sample")
    ap.add_argument("--cpu-decode-steps", type=int, default=8, help="decode steps per sampled request")
    ap.add_argument("--seed", type=int, default=4, help="seed of the GPU-drawn q/k/v")
    ap.add_argument("--no-shuffle", action="store_true", help="multi_turn_tree: hand out pool slots in order")
    ap.add_argument("--branch-chunk", type=int, default=1024,
                    help="classify_heavy: split size of the shared-prefix plan of the label branches")
    ap.add_argument("--branch-tiles", action="store_true",
                    help="classify_heavy: label branches on the extend tiles instead of the shared-prefix plan")
    ap.add_argument("--host-phases", action="store_true", help="report host wall time per phase of the last step")
    ap.add_argument("--page-size", type=int, default=1,
                    help="classify_heavy: KV pool pages of this many positions (the table then holds page ids)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run kv_store into contiguous slots (a plain copy of known size) and print its bytes; "
                         "the scale for rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return ap.parse_args()


class Phases:
    """Host wall time per phase of a step."""

    def __init__(self):
        self.ms, self.tick = {}, time.perf_counter()

    def start(self):
        self.tick = time.perf_counter()

    def mark(self, name):
        now = time.perf_counter()
        self.ms[name] = round((now - self.tick) * 1e3, 3)
        self.tick = now


def run_steps(args, one_step):
    """W untimed warm-up steps, then exactly K timed steps between device syncs;
    kernel times from the library's HIP events over the timed steps."""
    import torch

    import prefix_shared_kv_amd as pk
    for s in range(args.warmup):
        one_step(s)
    torch.cuda.synchronize()
    log(f"{args.warmup} warm-up steps done")
    pk.prof_collect()
    pk.prof_enable(True)
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_step(args.warmup + s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = pk.prof_collect()
    pk.prof_enable(False)
    log(f"{args.steps} timed steps done: {elapsed / args.steps * 1e3:.2f} ms/step")
    return elapsed, prof


def avg_ms(prof, name):
    return prof[name][1] / prof[name][0] if name in prof else 0.0


def extend_flops(D, Hq, P, E):
    """Causal-exact extend FLOPs: QK^T and PV over the visible keys only."""
    P = np.asarray(P, np.float64)
    E = np.asarray(E, np.float64)
    return 4.0 * D * Hq * float(np.sum(E * P + E * (E + 1) / 2.0))


def decode_bytes(pool_positions, B, Hq, Hkv, D):
    """Algorithmic bytes of one decode launch: every pool position on the
    batch's paths read once (K and V rows + its slot index), the current
    token's K/V read once and written to its slot (+ slot index), q and o."""
    row = 2 * Hkv * D * 2
    return pool_positions * (row + 4) + B * (2 * row + 4) + 2 * B * Hq * D * 2


def roofline(workload, name, bytes_per_launch, ms):
    gbs = bytes_per_launch / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(workload),
            "kernel": f"decode_attn_bf16<128> ({name})", "avg_launch_ms": round(ms, 5),
            "algorithmic_bytes_per_launch": float(bytes_per_launch), "traffic_unit": "bytes per launch"}


def extend_report(name, flops, ms, tokens):
    tf = flops / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    return {"kernel": name, "avg_launch_ms": round(ms, 4), "algorithmic_tflop": round(flops / 1e12, 4),
            "tflops": round(tf, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(tokens / (ms * 1e-3), 1) if ms > 0 else 0.0}


# ---------------------------------------------------------------------------
# classification + heavy decode
# ---------------------------------------------------------------------------
def bench_classify_heavy(args):
    import torch

    import prefix_shared_kv_amd as pk
    from prefix_shared_kv_amd import TokenBatch
    from prefix_shared_kv_amd.engine import Engine
    from synth import drive
    from synth import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # pieces of 4096 positions: 1024 long contexts give about two work units per
    # resident wave, and longer pieces start up fewer times
    args.chunk = args.chunk or 4096
    T = args.decode_steps or 8
    wc = W.classify64()
    wh = W.heavy_decode(n_decode=T)
    sh = wh.shape
    assert (wc.shape.num_q_heads, wc.shape.num_kv_heads, wc.shape.head_dim) == (sh.num_q_heads, sh.num_kv_heads,
                                                                                sh.head_dim)
    Hq, Hkv, D = sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    B = len(wh.requests)
    n_total = args.warmup + args.steps
    doc = wc.prefix_tokens(wc.requests[0])
    labels = [r.ext_tokens for r in wc.requests]
    n_lab = sum(len(x) for x in labels)
    cached = sum(len(n.tokens) for n in wh.nodes)
    # Steady-state pool: the decode contexts, one document with its branches and
    # the decode steps' slots.  From the second step on, the decode schedule
    # finds the pool short and evicts the least recently used unpinned nodes:
    # the previous step's branches and document (the decode contexts are
    # pinned by the batch that reads them).
    # With pages, every request also owns a partial page (a branch's label
    # tokens, the decode steps' tokens), so each needs up to a page more.
    ps = args.page_size
    pool = cached + (len(doc) + n_lab) + B * T + 1024 + (len(labels) + B) * (ps - 1)
    pool = -(-pool // ps) * ps
    kvs = pk.KVShape(Hq, Hkv, D, torch.bfloat16, pool, ps)
    base = np.array([len(wh.prompt_tokens(r)) for r in wh.requests], np.int32)
    stride = int(base.max()) + T + 8
    # Table rows for two steps' batches: rows are handed out oldest-free first,
    # so a step's batches never reuse rows whose uploads are still queued
    # behind the previous step's decode launches, and the host runs ahead.
    eng = Engine(kvs, stride, 2 * (B + len(wc.requests) + 8), dev)
    # The decode batch keeps its rows from step to step (two sets, used in
    # turn), as running requests do: rescheduled on its own rows, a request's
    # table row changes only in its last entries, and only those are uploaded.
    dec_rows = [eng.take_rows(B), eng.take_rows(B)]

    # ---- cached contexts of the decode requests (untimed set-up) ----
    drive.populate(eng, wh, device=dev, device_values=True)
    log(f"decode contexts cached: {cached} positions")

    # ---- inputs: token batches, q/k/v resident in HBM ----
    used = {int(n.tokens[0]) for n in wh.nodes if n.parent < 0}
    docs, nxt = [], int(doc[0])
    for _ in range(n_total):  # a fresh document per step: a first token no cached root edge starts with
        while nxt in used:
            nxt = (nxt + 1) % W.VOCAB
        used.add(nxt)
        d = doc.copy()
        d[0] = nxt
        docs.append(d)
    doc_tb = [TokenBatch([d]) for d in docs]
    br_tb = [TokenBatch([np.concatenate([d, lab]) for lab in labels]) for d in docs]
    hd_tb = TokenBatch([np.concatenate([wh.prompt_tokens(r), np.zeros(1, np.int32)]) for r in wh.requests])
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def randn(*s):
        return torch.randn(*s, device=dev, generator=gen, dtype=torch.float32).to(torch.bfloat16)

    L = len(doc)
    q_doc, k_doc, v_doc = randn(L, Hq, D), randn(L, Hkv, D), randn(L, Hkv, D)
    q_br, k_br, v_br = randn(n_lab, Hq, D), randn(n_lab, Hkv, D), randn(n_lab, Hkv, D)
    q_dec, k_dec, v_dec = randn(T, B, Hq, D), randn(T, B, Hkv, D), randn(T, B, Hkv, D)
    o_doc, o_br = torch.empty_like(q_doc), torch.empty_like(q_br)
    # next-token logits after each branch (one row per question, full vocabulary),
    # the 64 label tokens and the options of each question
    n_br = len(labels)
    logits = torch.from_numpy(W.next_token_logits(args.seed, n_br)).to(dev).to(torch.bfloat16)
    label_ids = torch.from_numpy(W.label_token_ids(args.seed)).to(dev)
    n_opts = torch.from_numpy(W.option_counts(args.seed, n_br)).to(dev)
    lab_out = (torch.empty(n_br, label_ids.numel(), device=dev), torch.empty(n_br, dtype=torch.int32, device=dev),
               torch.empty(n_br, device=dev), torch.empty(n_br, device=dev))
    o_dec = torch.empty(B, Hq, D, device=dev, dtype=torch.bfloat16)
    scale = wh.sm_scale
    plan_info, ph = {}, Phases()

    def one_step(s):
        ph.start()
        pk.prof_tag("prefill")
        bd = eng.schedule(doc_tb[s])
        eng.extend(bd, q_doc, k_doc, v_doc, scale, o=o_doc)
        eng.commit(bd)
        eng.release(bd)
        ph.mark("document")
        pk.prof_tag("branch")
        bb = eng.schedule(br_tb[s])
        eng.extend(bb, q_br, k_br, v_br, scale, o=o_br, cascade=not args.branch_tiles, chunk=args.branch_chunk)
        pk.label_distribution(logits, label_ids, n_opts, out=lab_out)
        eng.commit(bb)
        eng.release(bb)
        ph.mark("branches")
        pk.prof_tag(None)
        bh = eng.schedule(hd_tb, reserve=T - 1, rows=dec_rows[s % 2])
        ph.mark("decode_schedule")
        st = eng.prepare_decode(bh, base, T, chunk=args.chunk)
        plan_info.update(st.plan.summary)
        ph.mark("prepare_decode")
        for t in range(T):
            eng.decode_step(st, t, q_dec[t], k_dec[t], v_dec[t], scale, o=o_dec)
        ph.mark("decode_launches")
        eng.release(bh, keep=base)
        ph.mark("release")

    ev0 = eng.tree.stats()["evicted_tokens"]
    elapsed, prof = run_steps(args, one_step)
    evicted = eng.tree.stats()["evicted_tokens"] - ev0

    # ---- algorithmic work ----
    pre_flops = extend_flops(D, Hq, [0], [L])
    br_flops = extend_flops(D, Hq, [L] * len(labels), [len(x) for x in labels])
    pool_pos = cached + B * np.arange(T)  # every cached node once, plus the decode tokens already stored
    dec_bytes = float(np.mean(decode_bytes(pool_pos, B, Hq, Hkv, D)))
    row = 2 * Hkv * D * 2
    logical = float(np.mean(B * (base.mean() + np.arange(T) + 1)))  # positions the requests read, summed
    dec_name, mrg_name = "decode_attention_d128", "decode_merge"
    dec_ms, mrg_ms = avg_ms(prof, dec_name), avg_ms(prof, mrg_name)
    pre_ms = avg_ms(prof, "extend_bf16_d128@prefill")
    if args.branch_tiles:
        br_name, br_ms = "extend_bf16_d128@branch", avg_ms(prof, "extend_bf16_d128@branch")
    else:  # the shared-prefix plan: split-K launch + merge
        br_name = "extend_shared_d128@branch + extend_shared_merge@branch"
        br_ms = avg_ms(prof, "extend_shared_d128@branch") + avg_ms(prof, "extend_shared_merge@branch")
    tokens_per_step = L + n_lab + B * T
    res = {
        "metric": METRIC,
        "value": round(tokens_per_step * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded token trees; q/k/v N(0,1) drawn on the GPU)",
        "config": {
            "workload": "64-way single-token classification + heavy decode: GQA 32/4, head_dim 128, bf16; "
                        "a fresh 4096-token document prefilled and 64 label branches of 2-16 tokens extended over it; "
                        "1024 decode requests over 8192-token contexts (4096 shared per group of 16), 8 decode steps",
            "document_tokens": L, "branches": len(labels), "label_tokens": n_lab,
            "decode_batch": B, "decode_steps": T, "cached_positions": cached, "decode_chunk": args.chunk,
            "tokens_per_step": tokens_per_step, "pool_slots": pool, "page_size": ps,
        },
        "cache": {"evicted_tokens_per_step": round(evicted / n_total, 1)},
        "roofline": roofline("classify_heavy" if ps == 1 else f"classify_heavy_page{ps}", dec_name, dec_bytes, dec_ms),
        "extend": {
            "prefill": extend_report("extend_bf16_d128@prefill", pre_flops, pre_ms, L),
            "branches": extend_report(br_name, br_flops, br_ms, n_lab),
        },
        "labels": {"kernel": "label_distribution@branch", "avg_launch_ms": round(avg_ms(prof, "label_distribution@branch"), 5),
                   "questions": n_br, "labels": int(label_ids.numel())},
        "decode": {
            "attention_ms": round(dec_ms, 5), "merge_avg_ms": round(mrg_ms, 5),
            "unique_bytes_per_step": dec_bytes, "logical_bytes_per_step": logical * row,
            "effective_gbs": round(logical * row / (dec_ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(B / ((dec_ms + mrg_ms) * 1e-3), 1),
            "plan": {k: plan_info[k] for k in ("n_items", "shared_items", "max_splits")},
        },
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in prof.items()},
    }
    if args.host_phases:
        res["host_phase_ms"] = ph.ms
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_classify_heavy(wc, wh, args.cpu_sample, args.cpu_decode_steps,
                                                          tokens_per_step, T, args.seed)
    return res


def cpu_baseline_classify_heavy(wc, wh, n_req, n_dec, tokens_per_step, T, seed):
    """The float64 oracle, as it stands, on a bounded sample of one step: the
    document's prefill and the 64 branch extends in full, and the decode of
    `n_req` requests at `n_dec` of the T steps; the per-token decode time is
    scaled to the whole batch."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A
    from oracle import labels as LB
    from synth import workloads as W

    cores = len(os.sched_getaffinity(0))
    n_q = len(wc.requests)
    logits = W.next_token_logits(seed, n_q)
    label_ids, n_opts = W.label_token_ids(seed), W.option_counts(seed, n_q)
    pre = wc.prefill_nodes[0]
    q_doc = wc.node_prefill_q(pre)
    K_doc, V_doc = wc.node_kv(pre)
    branches = []
    for i in range(len(wc.requests)):
        q, k, v = wc.ext_qkv(i)
        branches.append((q, np.concatenate([K_doc, k]), np.concatenate([V_doc, v])))
    B = len(wh.requests)
    rids = sorted({int(x) for x in np.linspace(0, B - 1, n_req)})
    steps = sorted({int(x) for x in np.linspace(0, T - 1, n_dec)})
    ctx = {i: wh.context_kv(i, T) for i in rids}
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        A.extend(q_doc, K_doc, V_doc, 0, wc.sm_scale)
        t_pre = time.perf_counter() - t0
        t0 = time.perf_counter()
        for q, K, V in branches:
            A.extend(q, K, V, len(K_doc), wc.sm_scale)
        LB.classify(logits, label_ids, n_opts)
        t_br = time.perf_counter() - t0
        t_dec = 0.0
        for i in rids:
            K, V = ctx[i]
            base = len(K) - T
            for t in steps:
                q = wh.dec_qkv(i, t)[0]
                s = time.perf_counter()
                A.decode(q, K[:base + t + 1], V[:base + t + 1], wh.sm_scale)
                t_dec += time.perf_counter() - s
        n_tok = len(rids) * len(steps)
        t_dec /= n_tok
    est = t_pre + t_br + B * T * t_dec
    return {"value": round(tokens_per_step / est, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 numpy oracle on {cores} threads: the 4096-token prefill and the {len(branches)} branch "
                      f"extends and their label distributions in full, and {n_tok} decode tokens ({len(rids)} requests x {len(steps)} of the {T} "
                      f"steps); the decode time per token scaled to {B}x{T}: one step = {est:.1f} s",
            "sample_seconds": round(t_pre + t_br + n_tok * t_dec, 2)}


# ---------------------------------------------------------------------------
# multi-turn chat radix tree
# ---------------------------------------------------------------------------
def bench_multi_turn_tree(args):
    import torch

    import prefix_shared_kv_amd as pk
    from prefix_shared_kv_amd import TokenBatch
    from prefix_shared_kv_amd.engine import Engine
    from synth import drive
    from synth import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # pieces of 1024 positions: the tree's 256 requests give only about 1.3 work
    # units per resident wave at 4096, and the longest own ranges then end late
    args.chunk = args.chunk or 1024
    T = args.decode_steps or 256
    w = W.multi_turn_tree(n_decode=T)
    sh = w.shape
    Hq, Hkv, D = sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    B = len(w.requests)
    E = len(w.requests[0].ext_tokens)
    n_total = args.warmup + args.steps
    cached = sum(len(n.tokens) for n in w.nodes)
    pool = cached + n_total * B * E + B * (E + T) + 1024
    kvs = pk.KVShape(Hq, Hkv, D, torch.bfloat16, pool)
    stride = max(len(w.prompt_tokens(r)) for r in w.requests) + T + 8
    order = None if args.no_shuffle else np.random.default_rng(args.seed).permutation(pool).astype(np.int32)
    eng = Engine(kvs, stride, 2 * (B + 8), dev, free_order=order)  # two steps' rows, as above
    drive.populate(eng, w, device=dev, device_values=True)
    log("cached tree populated")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def randn(*s):
        return torch.randn(*s, device=dev, generator=gen, dtype=torch.float32).to(torch.bfloat16)

    q_ext, k_ext, v_ext = randn(B * E, Hq, D), randn(B * E, Hkv, D), randn(B * E, Hkv, D)
    q_dec, k_dec, v_dec = randn(T, B, Hq, D), randn(T, B, Hkv, D), randn(T, B, Hkv, D)
    o_ext = torch.empty_like(q_ext)
    o_dec = torch.empty(B, Hq, D, device=dev, dtype=torch.bfloat16)
    prefix = [w.prefix_tokens(r) for r in w.requests]

    def prompts(step):  # every step brings new tokens: the previous step's are cached by then
        out = []
        for r, p in zip(w.requests, prefix):
            e = r.ext_tokens.copy()
            e[0] = (int(e[0]) + step) % W.VOCAB
            out.append(np.concatenate([p, e]))
        return TokenBatch(out)

    batches = [prompts(s) for s in range(n_total)]
    plan_info, ph = {}, Phases()

    def one_step(s):
        ph.start()
        b = eng.schedule(batches[s], reserve=T)
        ph.mark("schedule")
        eng.extend(b, q_ext, k_ext, v_ext, w.sm_scale, o=o_ext)
        ph.mark("extend_launch")
        eng.commit(b)
        ph.mark("commit")
        st = eng.prepare_decode(b, b.tb.lens(), T, chunk=args.chunk)
        plan_info.update(st.plan.summary)
        ph.mark("prepare_decode")
        for t in range(T):
            eng.decode_step(st, t, q_dec[t], k_dec[t], v_dec[t], w.sm_scale, o=o_dec)
        ph.mark("decode_launches")
        eng.release(b)
        ph.mark("release")

    elapsed, prof = run_steps(args, one_step)

    P = np.array([len(p) for p in prefix], np.float64)
    ext_flops = extend_flops(D, Hq, P, [E] * B)
    pool_pos = cached + B * (E + np.arange(T))
    dec_bytes = float(np.mean(decode_bytes(pool_pos, B, Hq, Hkv, D)))
    row = 2 * Hkv * D * 2
    logical = float(np.mean(B * (P.mean() + E + np.arange(T) + 1)))
    dec_name, mrg_name = "decode_attention_d128", "decode_merge"
    dec_ms, mrg_ms, ext_ms = avg_ms(prof, dec_name), avg_ms(prof, mrg_name), avg_ms(prof, "extend_bf16_d128")
    tokens_per_step = B * E + B * T
    st_tot = prof["kv_store"][1] / args.steps if "kv_store" in prof else 0.0
    res = {
        "metric": METRIC,
        "value": round(tokens_per_step * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded token trees; q/k/v N(0,1) drawn on the GPU)",
        "config": {
            "workload": "multi-turn chat radix tree: GQA 32/8, head_dim 128, bf16, depth 4 x branching 4 "
                        "(340 cached segments, 256 leaf requests), segments U[256,1024], 128 new tokens "
                        "per leaf then 256 decode steps, shuffled pool slots",
            "batch": B, "new_tokens_per_request": E, "decode_steps": T, "cached_tokens": cached,
            "mean_prefix": round(float(P.mean()), 1), "decode_chunk": args.chunk,
            "slot_order": "in order" if args.no_shuffle else "shuffled", "tokens_per_step": tokens_per_step,
        },
        "roofline": roofline("multi_turn_tree", dec_name, dec_bytes, dec_ms),
        "extend": extend_report("extend_bf16_d128", ext_flops, ext_ms, B * E),
        "decode": {
            "attention_ms": round(dec_ms, 5), "merge_avg_ms": round(mrg_ms, 5),
            "unique_bytes_per_step": dec_bytes, "logical_bytes_per_step": logical * row,
            "effective_gbs": round(logical * row / (dec_ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(B / ((dec_ms + mrg_ms) * 1e-3), 1),
            "plan": {k: plan_info[k] for k in ("n_items", "shared_items", "max_splits")},
        },
        "kv_store": {"ms_per_step": round(st_tot, 4),
                     "gbs": round(B * E * (2 * row + 4) / (st_tot * 1e-3) / 1e9, 1) if st_tot else 0.0},
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in prof.items()},
    }
    if args.host_phases:
        res["host_phase_ms"] = ph.ms
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_tree(w, args.cpu_sample, args.cpu_decode_steps, tokens_per_step, T)
    return res


def cpu_baseline_tree(w, n_req, n_dec, tokens_per_step, T):
    """The float64 oracle, as it stands, on a bounded sample of one step: the
    extend of `n_req` requests and their decode at `n_dec` evenly spaced steps;
    the per-request extend time and per-token decode time are scaled to one step."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    cores = len(os.sched_getaffinity(0))
    rids = list(range(n_req))
    steps = sorted({int(x) for x in np.linspace(0, T - 1, n_dec)})
    ctx = {i: w.context_kv(i, T) for i in rids}
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for i in rids:
            K, V = ctx[i]
            P = len(w.prefix_tokens(w.requests[i]))
            q = w.ext_qkv(i)[0]
            A.extend(q, K[:P + len(q)], V[:P + len(q)], P, w.sm_scale)
        t_ext = (time.perf_counter() - t0) / n_req
        t_dec = 0.0
        for i in rids:
            K, V = ctx[i]
            base = len(K) - T
            for t in steps:
                q = w.dec_qkv(i, t)[0]
                s = time.perf_counter()
                A.decode(q, K[:base + t + 1], V[:base + t + 1], w.sm_scale)
                t_dec += time.perf_counter() - s
        t_dec /= len(steps) * n_req
    B = len(w.requests)
    est = B * t_ext + B * T * t_dec
    return {"value": round(tokens_per_step / est, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 numpy oracle on {cores} threads: extend of {n_req} requests (128 new tokens over "
                      f"their cached prefix) and their decode at {len(steps)} steps spread over 0..{T - 1}; "
                      f"scaled to one step ({B} extends + {B}x{T} decode tokens) = {est:.0f} s",
            "sample_seconds": round(n_req * t_ext + len(steps) * n_req * t_dec, 2)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path is a single-GPU kernel library measured on one MI355X; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.page_size != 1 and args.workload != "classify_heavy":
        print("--page-size applies to the classify_heavy workload", file=sys.stderr)
        sys.exit(2)
    res = bench_classify_heavy(args) if args.workload == "classify_heavy" else bench_multi_turn_tree(args)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
