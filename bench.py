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
The pool holds the 4.46M cached positions (9.1 GB of K and V); filling it with
one K/V scatter is timed apart from the step (pool_fill).

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

The other workloads share one step shape: a prefix (prefilled fresh every
step, or a cached tree) -> the requests' new tokens extended over it -> commit
-> decode steps -> release.
  --workload multi_turn_tree      GQA 32/8; a cached radix tree of depth 4 and
      branching 4 (340 segments of U[256,1024] tokens, 256 leaves), pool slots
      handed out in a seeded random order; 128 new tokens per leaf, 256 decode
      steps.
  --workload few_shot             GQA 32/8; a fresh 2048-token prefix prefilled,
      64 requests x 64 new tokens over it, 128 decode steps.
  --workload gpt2_system_prompt   12/12 heads, head_dim 64, inputs N(0,1)/8; a
      fresh 409-token system prompt prefilled, branches of 8 and 7 tokens,
      32 decode steps (latency-bound).
  --workload tiny_fp32            fp32, 4/4 heads, head_dim 64; a fresh
      128-token prefix, 2 requests x 8 new tokens, 4 decode steps (latency).

Inputs (q, k, v and the token batches) are made before timing; q, k and v
are drawn on the GPU and stay resident in HBM.  The K timed steps run without
kernel timing; K more steps then bracket every library kernel with HIP events
for the per-kernel durations (the roofline figures), since recording events
costs each launch a few microseconds that would count in the step time of the
launch-bound workloads.  The cpu_baseline leg runs the float64 oracle on host
copies of those same inputs, times it, and compares the outputs of the last
step with it (error histogram).
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
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, TFLOP/s
# the path's targets: extend at half the dense bf16 MFMA peak, decode at 0.7 of the HBM peak
TARGET_EXTEND_MFMA_FRAC = 0.50
TARGET_DECODE_HBM_FRAC = 0.70


def targets(extend_fracs, decode_frac, decode_hbm=True):
    """Each target beside what this run measured and whether it is met."""
    out = {"extend_bf16_mfma_frac": {"target": TARGET_EXTEND_MFMA_FRAC, "measured": extend_fracs,
                                     "met": all(f >= TARGET_EXTEND_MFMA_FRAC for f in extend_fracs.values())}}
    if decode_hbm:
        out["decode_hbm_frac"] = {"target": TARGET_DECODE_HBM_FRAC, "measured": decode_frac,
                                  "met": decode_frac >= TARGET_DECODE_HBM_FRAC}
    else:
        out["decode_hbm_frac"] = {"target": TARGET_DECODE_HBM_FRAC, "measured": None, "met": None,
                                  "note": "the decode working set fits the Infinity Cache: not an HBM-bound figure"}
    return out
ROOT = os.path.dirname(os.path.abspath(__file__))
# what the decode kernel's code depends on: its sources and the build flags;
# a traffic figure stands only while these are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "prefix_shared_kv_amd", "csrc", f)
                  for f in ("decode.hip", "attn_tile.h", "hip_common.h")] + [
                  os.path.join(ROOT, "prefix_shared_kv_amd", "build.py")]
METRIC = "extend-attn TFLOP/s (% MFMA peak) + decode-attn HBM GB/s, tokens/s, 1 GPU"
WORKLOADS = ("classify_heavy", "multi_turn_tree", "few_shot", "gpt2_system_prompt", "tiny_fp32")
# absolute-error bins of the histogram against the oracle (upper edges)
ERR_EDGES = (1e-4, 1e-3, 4e-3, 1e-2, 2e-2)


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


def ceilings():
    """Measured ceilings beside the datasheet peaks (libceilings.so): a streaming
    read of 8 GiB with plain and with nontemporal 16-byte loads, 1024 and 2048
    waves each streaming its own contiguous 512 KiB, the K/V scatter
    as a copy of 2 x 4.3 GB into contiguous slots, and a dense loop of
    v_mfma_f32_32x32x16_bf16 (four independent chains per wave, two waves per SIMD)."""
    import ctypes as C

    import torch

    import prefix_shared_kv_amd as pk
    lib = C.CDLL(os.path.join(ROOT, "prefix_shared_kv_amd", "libceilings.so"))
    lib.ceil_stream_read_ms.restype = C.c_double
    lib.ceil_stream_read_ms.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    lib.ceil_mfma_ms.restype = C.c_double
    lib.ceil_mfma_ms.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    dev = torch.device("cuda:0")
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    word = torch.zeros(4, dtype=torch.int32, device=dev)
    out = {"peaks": {"hbm_gbs": HBM_PEAK_GBS, "mfma_bf16_tflops": MFMA_BF16_PEAK_TFLOPS}}
    n = 8 << 30
    buf = torch.full((n,), 1, dtype=torch.uint8, device=dev)
    for nt in (0, 1):
        ms = lib.ceil_stream_read_ms(C.c_void_p(buf.data_ptr()), n, nt, 5, C.c_void_p(word.data_ptr()), stream)
        if ms <= 0:
            raise RuntimeError(f"stream read failed ({ms})")
        out["stream_read_nontemporal" if nt else "stream_read"] = {
            "bytes": n, "avg_ms": round(ms, 4), "gbs": round(n / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # each wave streaming its own contiguous 512 KiB (16 KiB per wave in flight)
    word2 = torch.zeros(4, dtype=torch.int32, device=dev)
    lib.ceil_wave_stream_ms.restype = C.c_double
    lib.ceil_wave_stream_ms.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    per_wave = 512 << 10
    for waves in (1024, 2048):
        assert waves * per_wave <= n
        ms = lib.ceil_wave_stream_ms(C.c_void_p(buf.data_ptr()), waves, per_wave // 16384, 5,
                                     C.c_void_p(word2.data_ptr()), stream)
        if ms <= 0:
            raise RuntimeError(f"wave stream failed ({ms})")
        nb = waves * per_wave
        out[f"wave_stream_{waves}"] = {
            "bytes": nb, "waves": waves, "avg_ms": round(ms, 4), "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del buf
    torch.cuda.empty_cache()
    # the scatter as a plain copy: 2.1M rows of 8 x 128 bf16 (K and V) into contiguous slots
    rows, h, d = 1 << 21, 8, 128
    kvs = pk.KVShape(32, h, d, torch.bfloat16, rows)
    pool_k = torch.empty((rows, h, d), dtype=torch.bfloat16, device=dev)
    pool_v = torch.empty_like(pool_k)
    src_k = torch.ones_like(pool_k)
    src_v = torch.ones_like(pool_k)
    slots = torch.arange(rows, dtype=torch.int32, device=dev)
    pk.kv_store(kvs, pool_k, pool_v, src_k, src_v, slots)
    torch.cuda.synchronize()
    pk.prof_collect()
    pk.prof_enable(True)
    for _ in range(5):
        pk.kv_store(kvs, pool_k, pool_v, src_k, src_v, slots)
    torch.cuda.synchronize()
    prof = pk.prof_collect()
    pk.prof_enable(False)
    ms = avg_ms(prof, "kv_store")
    nbytes = 2 * (2 * rows * h * d * 2) + 4 * rows
    out["copy_kv_store"] = {"bytes_moved": nbytes, "avg_ms": round(ms, 4), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                            "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del pool_k, pool_v, src_k, src_v, slots
    torch.cuda.empty_cache()
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks, iters = 2 * cu, 8192
    ms = lib.ceil_mfma_ms(blocks, iters, 5, C.c_void_p(word.data_ptr()), stream)
    if ms <= 0:
        raise RuntimeError(f"mfma loop failed ({ms})")
    flops = blocks * 4 * 4 * iters * 32768.0
    tf = flops / (ms * 1e-3) / 1e12
    out["mfma_bf16_32x32x16"] = {"workgroups": blocks, "waves_per_simd": 2, "flops": flops, "avg_ms": round(ms, 4),
                                 "tflops": round(tf, 1), "frac_of_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                 "implied_clock_ghz_at_full_rate": round(tf * 1e12 / (cu * 4 * 1024) / 1e9, 3)}
    print(json.dumps({"ceilings": out}))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=WORKLOADS, default="classify_heavy")
    ap.add_argument("--chunk", type=int, default=None,
                    help="decode split size, nominal positions per work item (default: 4096 for classify_heavy, "
                         "1024 for multi_turn_tree, sized from the step for the small workloads)")
    ap.add_argument("--decode-steps", type=int, default=None, help="decode steps per step (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time the oracle's sample may take: requests are added until it is spent")
    ap.add_argument("--cpu-decode-steps", type=int, default=8, help="decode steps per sampled request")
    ap.add_argument("--seed", type=int, default=4, help="seed of the GPU-drawn q/k/v")
    ap.add_argument("--no-shuffle", action="store_true", help="multi_turn_tree: hand out pool slots in order")
    ap.add_argument("--branch-chunk", type=int, default=None,
                    help="classify_heavy: split size of the shared-prefix plan of the label branches "
                         "(default: sized to fill the GPU once)")
    ap.add_argument("--branch-tiles", action="store_true",
                    help="classify_heavy: label branches on the extend tiles instead of the shared-prefix plan")
    ap.add_argument("--cascade", action="store_true",
                    help="tree workloads: the requests' extend over a shared-prefix plan instead of the tiles")
    ap.add_argument("--host-phases", action="store_true", help="report host wall time per phase of the last step")
    ap.add_argument("--page-size", type=int, default=1,
                    help="classify_heavy: KV pool pages of this many positions (the table then holds page ids)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the streaming-read, copy and MFMA-loop ceilings and print them")
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
    """W untimed warm-up steps, then exactly K timed steps between device syncs,
    whose wall time is the step time; then K more steps with every library
    kernel bracketed by HIP events on its stream, for the per-kernel durations.
    Recording the events costs each launch a few microseconds of host and GPU
    time, which the step time of a launch-bound workload must not include."""
    import torch

    import prefix_shared_kv_amd as pk
    for s in range(args.warmup):
        one_step(s)
    torch.cuda.synchronize()
    log(f"{args.warmup} warm-up steps done")
    pk.prof_collect()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_step(args.warmup + s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"{args.steps} timed steps done: {elapsed / args.steps * 1e3:.2f} ms/step")
    pk.prof_enable(True)
    for s in range(args.steps):
        one_step(args.warmup + args.steps + s)
    torch.cuda.synchronize()
    prof = pk.prof_collect()
    pk.prof_enable(False)
    log(f"{args.steps} steps with kernel timing done")
    return elapsed, prof


def avg_ms(prof, name):
    return prof[name][1] / prof[name][0] if name in prof else 0.0


def extend_flops(D, Hq, P, E):
    """Causal-exact extend FLOPs: QK^T and PV over the visible keys only."""
    P = np.asarray(P, np.float64)
    E = np.asarray(E, np.float64)
    return 4.0 * D * Hq * float(np.sum(E * P + E * (E + 1) / 2.0))


def decode_bytes(pool_positions, B, Hq, Hkv, D, elem=2):
    """Algorithmic bytes of one decode launch: every pool position on the
    batch's paths read once (K and V rows + its slot index), the current
    token's K/V read once and written to its slot (+ slot index), q and o."""
    row = 2 * Hkv * D * elem
    return pool_positions * (row + 4) + B * (2 * row + 4) + 2 * B * Hq * D * elem


def roofline(workload, name, bytes_per_launch, ms):
    gbs = bytes_per_launch / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(workload),
            "kernel": name, "avg_launch_ms": round(ms, 5),
            "algorithmic_bytes_per_launch": float(bytes_per_launch), "traffic_unit": "bytes per launch"}


def extend_report(name, flops, ms, tokens, peak=MFMA_BF16_PEAK_TFLOPS):
    tf = flops / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    return {"kernel": name, "avg_launch_ms": round(ms, 4), "algorithmic_tflop": round(flops / 1e12, 6),
            "tflops": round(tf, 2), "peak_tflops": peak, "frac": round(tf / peak, 4),
            "tokens_per_s": round(tokens / (ms * 1e-3), 1) if ms > 0 else 0.0}


def host64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class ErrorHistogram:
    """Element-wise absolute errors of GPU outputs against the oracle, binned."""

    def __init__(self):
        self.counts = np.zeros(len(ERR_EDGES) + 1, np.int64)
        self.max = 0.0
        self.n = 0

    def add(self, got, want):
        e = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64)).ravel()
        self.counts += np.bincount(np.searchsorted(ERR_EDGES, e, side="left"), minlength=len(ERR_EDGES) + 1)
        self.max = max(self.max, float(e.max()) if e.size else 0.0)
        self.n += e.size

    def report(self):
        names = [f"<={x:g}" for x in ERR_EDGES] + [f">{ERR_EDGES[-1]:g}"]
        return {"max_abs": self.max, "elements": int(self.n), "bins": dict(zip(names, self.counts.tolist()))}


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
    n_total = args.warmup + 2 * args.steps  # the timed steps, then as many with kernel timing
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

    # ---- pool fill: one K/V scatter of every pool row (timed apart) ----
    fill = pool_fill(kvs, eng, dev)
    log(f"pool fill: {fill['avg_launch_ms']:.3f} ms per launch, {fill['achieved']:.0f} GB/s")

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
    o_dec = torch.empty(T, B, Hq, D, device=dev, dtype=torch.bfloat16)  # every decode step's outputs
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
            eng.decode_step(st, t, q_dec[t], k_dec[t], v_dec[t], scale, o=o_dec[t])
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
            "branch_chunk": args.branch_chunk or "sized to fill the GPU once",
            "tokens_per_step": tokens_per_step, "pool_slots": pool, "page_size": ps,
        },
        "cache": {"evicted_tokens_per_step": round(evicted / n_total, 1)},
        "roofline": roofline("classify_heavy" if ps == 1 else f"classify_heavy_page{ps}",
                             f"decode_attn_bf16<128> ({dec_name})", dec_bytes, dec_ms),
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
        "pool_fill": fill,
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in prof.items()},
    }
    res["targets"] = targets({"prefill": res["extend"]["prefill"]["frac"], "branches": res["extend"]["branches"]["frac"]},
                             res["roofline"]["frac"])
    if args.host_phases:
        res["host_phase_ms"] = ph.ms
    if not args.no_cpu_baseline:
        gpu = dict(q_doc=q_doc, k_doc=k_doc, v_doc=v_doc, o_doc=o_doc, q_br=q_br, k_br=k_br, v_br=v_br, o_br=o_br,
                   q_dec=q_dec, k_dec=k_dec, v_dec=v_dec, o_dec=o_dec)
        res["cpu_baseline"], res["error"] = cpu_baseline_classify_heavy(
            wc, wh, gpu, args.cpu_seconds, args.cpu_decode_steps, tokens_per_step, T, dev)
    return res


def pool_fill(kvs, eng, dev, reps=3):
    """One rc_kv_store of every pool row (K and V from a scratch source, slots in
    order), timed with the library's HIP events; the pool is filled properly
    afterwards.  Algorithmic bytes = new rows read + pool rows written + slot list."""
    import torch

    import prefix_shared_kv_amd as pk
    S = kvs.pool_slots
    k = torch.randn(S, kvs.num_kv_heads, kvs.head_dim, device=dev).to(kvs.dtype)
    v = torch.randn_like(k)
    slots = torch.arange(S, dtype=torch.int32, device=dev)
    pk.kv_store(kvs, eng.k_pool, eng.v_pool, k, v, slots)  # warm-up
    torch.cuda.synchronize()
    pk.prof_collect()
    pk.prof_enable(True)
    pk.prof_tag("fill")
    for _ in range(reps):
        pk.kv_store(kvs, eng.k_pool, eng.v_pool, k, v, slots)
    torch.cuda.synchronize()
    prof = pk.prof_collect()
    pk.prof_enable(False)
    pk.prof_tag(None)
    ok = bool(torch.equal(eng.k_pool, k) and torch.equal(eng.v_pool, v))
    del k, v, slots
    torch.cuda.empty_cache()
    ms = avg_ms(prof, "kv_store@fill")
    row = 2 * kvs.num_kv_heads * kvs.head_dim * (4 if kvs.dtype == torch.float32 else 2)
    nbytes = 2 * S * row + 4 * S
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "kv_store_kernel", "rows": S, "launches": reps, "avg_launch_ms": round(ms, 4),
            "algorithmic_bytes_per_launch": float(nbytes), "achieved": round(gbs, 1), "unit": "GB/s",
            "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4), "bit_exact": ok}


def cpu_baseline_classify_heavy(wc, wh, gpu, budget, n_dec, tokens_per_step, T, dev):
    """The float64 oracle, as it stands, on a bounded sample of one step, over
    host copies of the step's own inputs: the document's prefill and the 64
    branch extends in full, then the decode of requests (in a seeded order) at
    `n_dec` of the T steps, their contexts regenerated from the seeded node
    draws, until `budget` seconds of oracle time are spent; the per-token decode
    time is scaled to the whole batch.  The last step's GPU outputs for
    the same items give the error histogram."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    cores = len(os.sched_getaffinity(0))
    h = {k: host64(v) for k, v in gpu.items() if k != "o_dec"}
    q_doc, K_doc, V_doc = h["q_doc"], h["k_doc"], h["v_doc"]
    lens = [len(r.ext_tokens) for r in wc.requests]
    starts = np.concatenate([[0], np.cumsum(lens)])
    branches = [(h["q_br"][a:b], np.concatenate([K_doc, h["k_br"][a:b]]), np.concatenate([V_doc, h["v_br"][a:b]]))
                for a, b in zip(starts[:-1], starts[1:])]
    B = len(wh.requests)
    order = np.random.default_rng(0).permutation(B)
    steps = sorted({int(x) for x in np.linspace(0, T - 1, min(n_dec, T))})
    node_cache = {}

    def node(nid):
        if nid not in node_cache:
            k, v = wh.node_kv_device(nid, dev)
            node_cache[nid] = (host64(k), host64(v))
        return node_cache[nid]

    def context(i):
        r = wh.requests[i]
        K = np.concatenate([node(n)[0] for n in r.path] + [h["k_dec"][:, i]])
        V = np.concatenate([node(n)[1] for n in r.path] + [h["v_dec"][:, i]])
        return K, V

    o_dec = {t: host64(gpu["o_dec"][t]) for t in steps}
    hist = {"prefill": ErrorHistogram(), "branches": ErrorHistogram(), "decode": ErrorHistogram()}
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        want = A.extend(q_doc, K_doc, V_doc, 0, wc.sm_scale)
        t_pre = time.perf_counter() - t0
        hist["prefill"].add(host64(gpu["o_doc"]), want)
        t_br = 0.0
        o_br = host64(gpu["o_br"])
        for (q, K, V), a, b in zip(branches, starts[:-1], starts[1:]):
            t0 = time.perf_counter()
            want = A.extend(q, K, V, len(K_doc), wc.sm_scale)
            t_br += time.perf_counter() - t0
            hist["branches"].add(o_br[a:b], want)
        t_dec, n_req = 0.0, 0
        for i in order:
            if n_req and t_pre + t_br + t_dec >= budget:
                break
            K, V = context(int(i))
            base = len(K) - T
            for t in steps:
                s = time.perf_counter()
                want = A.decode(h["q_dec"][t, i], K[:base + t + 1], V[:base + t + 1], wh.sm_scale)
                t_dec += time.perf_counter() - s
                hist["decode"].add(o_dec[t][i], want)
            n_req += 1
        n_tok = n_req * len(steps)
        t_dec /= n_tok
    est = t_pre + t_br + B * T * t_dec
    cpu = {"value": round(tokens_per_step / est, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"float64 numpy oracle on {cores} threads: the 4096-token prefill and the {len(branches)} branch "
                     f"extends in full, and {n_tok} decode tokens ({n_req} requests x {len(steps)} of the {T} "
                     f"steps); the decode time per token scaled to {B}x{T}: one step = {est:.1f} s",
           "sample_seconds": round(t_pre + t_br + n_tok * t_dec, 2)}
    err = {k: v.report() for k, v in hist.items()}
    err["compared"] = "the last step's outputs (the last step with kernel timing) over the oracle's sample, element-wise"
    return cpu, err


# ---------------------------------------------------------------------------
# tree-shaped workloads: a prefix (prefilled every step, or a cached tree),
# the requests' extend over it, commit, decode steps, release
# ---------------------------------------------------------------------------
TREE_SPECS = {
    "multi_turn_tree": dict(
        make=lambda W, T: W.multi_turn_tree(n_decode=T), decode_steps=256, chunk=1024,
        text="multi-turn chat radix tree: GQA 32/8, head_dim 128, bf16, depth 4 x branching 4 (340 cached "
             "segments, 256 leaf requests), segments U[256,1024], 128 new tokens per leaf then 256 decode steps, "
             "shuffled pool slots"),
    "few_shot": dict(
        make=lambda W, T: W.few_shot(n_decode=T), decode_steps=128, chunk=None,
        text="few-shot batch: GQA 32/8, head_dim 128, bf16; a fresh 2048-token prefix prefilled each step, "
             "64 requests x 64 new tokens extended over it, then 128 decode steps"),
    "gpt2_system_prompt": dict(
        make=lambda W, T: W.gpt2_system_prompt(), decode_steps=32, chunk=None,
        text="GPT-2-small-shaped layer: 12/12 heads, head_dim 64, bf16, inputs N(0,1)/8; a fresh 409-token system "
             "prompt prefilled each step, branches of 8 and 7 tokens, 32 decode steps each"),
    "tiny_fp32": dict(
        make=lambda W, T: W.tiny_fp32(), decode_steps=4, chunk=None,
        text="tiny single-layer attention, fp32: 4/4 heads, head_dim 64; a fresh 128-token prefix prefilled each "
             "step, 2 requests x 8 new tokens, 4 decode steps"),
}


def bench_tree(args):
    import torch

    import prefix_shared_kv_amd as pk
    from prefix_shared_kv_amd import TokenBatch
    from prefix_shared_kv_amd.engine import Engine
    from synth import drive
    from synth import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = TREE_SPECS[args.workload]
    args.chunk = args.chunk or spec["chunk"]
    T = args.decode_steps or spec["decode_steps"]
    w = spec["make"](W, T)
    sh = w.shape
    Hq, Hkv, D = sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    f32 = sh.dtype == "f32"
    dt = torch.float32 if f32 else torch.bfloat16
    elem = 4 if f32 else 2
    reqs = w.requests
    B = len(reqs)
    E = np.array([len(r.ext_tokens) for r in reqs], np.int64)
    n_total = args.warmup + 2 * args.steps  # the timed steps, then as many with kernel timing
    prefill = list(w.prefill_nodes)          # prefilled fresh every step
    fresh = bool(prefill)
    cached_nodes = [n for n in drive.node_order(w) if n not in prefill]
    cached = sum(len(w.nodes[n].tokens) for n in cached_nodes)
    pre_tokens = sum(len(w.nodes[n].tokens) for n in prefill)
    # pool: the cached tree, the decode slots, and the prefixes and new tokens of
    # two steps (every step brings new tokens; when the pool runs short the
    # schedule evicts the least recently used unpinned nodes: earlier steps');
    # with a cached tree and no eviction, every step's new tokens stay cached
    pool = cached + (2 if fresh else n_total) * (pre_tokens + int(E.sum())) + B * T + 1024
    kvs = pk.KVShape(Hq, Hkv, D, dt, pool)
    prompt_len = np.array([len(w.prompt_tokens(r)) for r in reqs], np.int32)
    stride = int(prompt_len.max()) + T + 8
    order = None
    if w.shuffle_slots and not args.no_shuffle:
        order = np.random.default_rng(args.seed).permutation(pool).astype(np.int32)
    eng = Engine(kvs, stride, 2 * (B + len(prefill) + 8), dev, free_order=order)  # two steps' rows
    if cached_nodes:
        drive.populate(eng, w, cached_nodes, device=dev, device_values=True)
        log(f"cached tree populated: {cached} positions")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def randn(*s):
        x = torch.randn(*s, device=dev, generator=gen, dtype=torch.float32)
        return (x * sh.std if sh.std != 1.0 else x).to(dt)

    q_pre = {n: randn(len(w.nodes[n].tokens), Hq, D) for n in prefill}
    k_pre = {n: randn(len(w.nodes[n].tokens), Hkv, D) for n in prefill}
    v_pre = {n: randn(len(w.nodes[n].tokens), Hkv, D) for n in prefill}
    o_pre = {n: torch.empty_like(q_pre[n]) for n in prefill}
    n_ext = int(E.sum())
    q_ext, k_ext, v_ext = randn(n_ext, Hq, D), randn(n_ext, Hkv, D), randn(n_ext, Hkv, D)
    q_dec, k_dec, v_dec = randn(T, B, Hq, D), randn(T, B, Hkv, D), randn(T, B, Hkv, D)
    o_ext = torch.empty_like(q_ext)
    o_dec = torch.empty(T, B, Hq, D, device=dev, dtype=dt)

    # every step brings new tokens: a fresh first token for each prefilled root
    # (then nothing of the prompts is cached), or a new first token of each
    # request's own tokens over the cached tree
    used = {int(n.tokens[0]) for n in w.nodes if n.parent < 0}
    node_tok = []
    nxt = 1
    for s in range(n_total):
        toks = {n.id: n.tokens for n in w.nodes}
        for nid in prefill:
            if w.nodes[nid].parent < 0:
                while nxt in used:
                    nxt = (nxt + 1) % W.VOCAB
                used.add(nxt)
                t = w.nodes[nid].tokens.copy()
                t[0] = nxt
                toks[nid] = t
        node_tok.append(toks)

    def path_tokens(s, nid):
        ids = []
        while nid >= 0:
            ids.append(nid)
            nid = w.nodes[nid].parent
        return np.concatenate([node_tok[s][i] for i in reversed(ids)]).astype(np.int32)

    def prompts(s):
        out = []
        for r in reqs:
            e = r.ext_tokens.copy()
            if not fresh and len(e):
                e[0] = (int(e[0]) + s) % W.VOCAB
            pre = path_tokens(s, r.path[-1]) if r.path else np.zeros(0, np.int32)
            out.append(np.concatenate([pre, e]).astype(np.int32))
        return TokenBatch(out)

    pre_tb = [{n: TokenBatch([path_tokens(s, n)]) for n in prefill} for s in range(n_total)]
    req_tb = [prompts(s) for s in range(n_total)]
    P_expect = np.array([len(w.prefix_tokens(r)) for r in reqs], np.int32)
    scale = w.sm_scale
    plan_info, ph, seen = {}, Phases(), {}

    def one_step(s):
        ph.start()
        pk.prof_tag("prefill")
        for nid in prefill:
            b = eng.schedule(pre_tb[s][nid])
            eng.extend(b, q_pre[nid], k_pre[nid], v_pre[nid], scale, o=o_pre[nid])
            eng.commit(b)
            eng.release(b)
        ph.mark("prefill")
        pk.prof_tag("extend")
        b = eng.schedule(req_tb[s], reserve=T)
        seen["P"] = b.prefix_lens.copy()
        ph.mark("schedule")
        eng.extend(b, q_ext, k_ext, v_ext, scale, o=o_ext, cascade=args.cascade)
        ph.mark("extend_launch")
        eng.commit(b)
        ph.mark("commit")
        pk.prof_tag(None)
        st = eng.prepare_decode(b, prompt_len, T, chunk=args.chunk)
        plan_info.update(st.plan.summary)
        plan_info["chunk"] = st.plan.info.chunk
        ph.mark("prepare_decode")
        for t in range(T):
            eng.decode_step(st, t, q_dec[t], k_dec[t], v_dec[t], scale, o=o_dec[t])
        ph.mark("decode_launches")
        eng.release(b)
        ph.mark("release")

    elapsed, prof = run_steps(args, one_step)
    if not np.array_equal(seen["P"], P_expect):
        raise RuntimeError(f"matched prefixes {seen['P'][:8]} differ from the workload's {P_expect[:8]}")

    # ---- algorithmic work ----
    dtag = "d128" if D == 128 else "d64"
    kind = "f32" if f32 else "bf16"
    ext_name = f"extend_shared_{dtag}@extend" if args.cascade else f"extend_{kind}_{dtag}@extend"
    ext_ms = avg_ms(prof, ext_name) + (avg_ms(prof, "extend_shared_merge@extend") if args.cascade else 0.0)
    pre_name = f"extend_{kind}_{dtag}@prefill"
    pre_ms = avg_ms(prof, pre_name)
    peak = FP32_VECTOR_PEAK_TFLOPS if f32 else MFMA_BF16_PEAK_TFLOPS
    pre_flops = sum(extend_flops(D, Hq, [w.node_start(n)], [len(w.nodes[n].tokens)]) for n in prefill)
    ext_flops = extend_flops(D, Hq, P_expect, E)
    dec_name = f"decode_f32_{dtag}" if f32 else f"decode_attention_{dtag}"
    dec_ms, mrg_ms = avg_ms(prof, dec_name), avg_ms(prof, "decode_merge")
    path_nodes = {n for r in reqs for n in r.path}
    shared_pos = sum(len(w.nodes[n].tokens) for n in path_nodes)
    pool_pos = shared_pos + n_ext + B * np.arange(T)  # tree positions once, own tokens, earlier decode tokens
    dec_bytes = float(np.mean(decode_bytes(pool_pos, B, Hq, Hkv, D, elem)))
    row = 2 * Hkv * D * elem
    logical = float(np.mean(B * (prompt_len.mean() + np.arange(T) + 1)))
    tokens_per_step = pre_tokens + n_ext + B * T
    st_ms = prof["kv_store@extend"][1] / args.steps if "kv_store@extend" in prof else 0.0
    res = {
        "metric": METRIC,
        "value": round(tokens_per_step * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32" if f32 else "bf16",
        "data": "synthetic (seeded token trees; q/k/v drawn on the GPU)",
        "config": {
            "workload": spec["text"],
            "batch": B, "new_tokens": n_ext, "prefill_tokens": pre_tokens, "decode_steps": T,
            "cached_tokens": cached, "mean_prefix": round(float(P_expect.mean()), 1),
            "decode_chunk": args.chunk or f"{plan_info['chunk']} (sized from the step)",
            "extend_path": "shared-prefix plan" if args.cascade else "tiles",
            "slot_order": "shuffled" if order is not None else "in order", "tokens_per_step": tokens_per_step,
        },
        "roofline": roofline(args.workload, dec_name, dec_bytes, dec_ms),
        "extend": extend_report(ext_name, ext_flops, ext_ms, n_ext, peak),
        "decode": {
            "attention_ms": round(dec_ms, 5), "merge_avg_ms": round(mrg_ms, 5),
            "unique_bytes_per_step": dec_bytes, "logical_bytes_per_step": logical * row,
            "effective_gbs": round(logical * row / (dec_ms * 1e-3) / 1e9, 1) if dec_ms else 0.0,
            "tokens_per_s": round(B / ((dec_ms + mrg_ms) * 1e-3), 1) if dec_ms else 0.0,
            "plan": {k: plan_info[k] for k in ("n_items", "shared_items", "max_splits")},
        },
        "kv_store": {"ms_per_step": round(st_ms, 4),
                     "gbs": round(n_ext * (2 * row + 4) / (st_ms * 1e-3) / 1e9, 1) if st_ms else 0.0},
        "latency_ms": {"prefill": round(pre_ms, 5), "extend": round(ext_ms, 5),
                       "decode_step": round(dec_ms + mrg_ms, 5), "step": round(elapsed / args.steps * 1e3, 3)},
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in prof.items()},
    }
    if prefill:
        res["prefill"] = extend_report(pre_name, pre_flops, pre_ms, pre_tokens, peak)
    if dec_bytes < 256e6:  # the decode working set fits the 256 MB Infinity Cache
        res["roofline"]["note"] = ("decode working set below the 256 MB Infinity Cache: served from it across "
                                   "steps, so GB/s here is not HBM evidence")
    if not f32:  # the targets are for the bf16 path
        fr = {"extend": res["extend"]["frac"]}
        if prefill:
            fr["prefill"] = res["prefill"]["frac"]
        res["targets"] = targets(fr, res["roofline"]["frac"], decode_hbm=dec_bytes >= 256e6)
    if args.host_phases:
        res["host_phase_ms"] = ph.ms
    if not args.no_cpu_baseline:
        gpu = dict(q_pre=q_pre, k_pre=k_pre, v_pre=v_pre, o_pre=o_pre, q_ext=q_ext, k_ext=k_ext, v_ext=v_ext,
                   o_ext=o_ext, q_dec=q_dec, k_dec=k_dec, v_dec=v_dec, o_dec=o_dec)
        res["cpu_baseline"], res["error"] = cpu_baseline_tree(w, gpu, args.cpu_seconds, args.cpu_decode_steps,
                                                              tokens_per_step, T, dev)
    return res


def cpu_baseline_tree(w, gpu, budget, n_dec, tokens_per_step, T, dev):
    """The float64 oracle, as it stands, on a bounded sample of one step, over
    host copies of the step's own inputs: up to 64 evenly spaced rows of each
    prefilled prefix, then requests in a seeded order (their extend and their
    decode at `n_dec` evenly spaced steps, contexts from the seeded node draws)
    until `budget` seconds of oracle time are spent; the per-row, per-request
    and per-token times are scaled to one step.  The last step's GPU
    outputs for the same items give the error histogram."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    cores = len(os.sched_getaffinity(0))
    reqs = w.requests
    B = len(reqs)
    E = [len(r.ext_tokens) for r in reqs]
    starts = np.concatenate([[0], np.cumsum(E)])
    order = np.random.default_rng(0).permutation(B)
    steps = sorted({int(x) for x in np.linspace(0, T - 1, min(n_dec, T))})
    q_ext, k_ext, v_ext = (host64(gpu[k]) for k in ("q_ext", "k_ext", "v_ext"))
    q_dec, k_dec, v_dec = (host64(gpu[k]) for k in ("q_dec", "k_dec", "v_dec"))
    o_ext = host64(gpu["o_ext"])
    o_dec = {t: host64(gpu["o_dec"][t]) for t in steps}
    nodes = {}
    for n in w.prefill_nodes:
        nodes[n] = (host64(gpu["k_pre"][n]), host64(gpu["v_pre"][n]))

    def node(nid):
        if nid not in nodes:
            k, v = w.node_kv_device(nid, dev)
            nodes[nid] = (host64(k), host64(v))
        return nodes[nid]

    def context(i):
        r = reqs[i]
        ks = [node(n)[0] for n in r.path] + [k_ext[starts[i]:starts[i + 1]], k_dec[:, i]]
        vs = [node(n)[1] for n in r.path] + [v_ext[starts[i]:starts[i + 1]], v_dec[:, i]]
        return np.concatenate(ks), np.concatenate(vs)

    def path_kv(nid):
        ids = []
        while nid >= 0:
            ids.append(nid)
            nid = w.nodes[nid].parent
        kv = [node(i) for i in reversed(ids)]
        return np.concatenate([k for k, _ in kv]), np.concatenate([v for _, v in kv])

    hist = {"prefill": ErrorHistogram(), "extend": ErrorHistogram(), "decode": ErrorHistogram()}
    t_pre = t_pre_sampled = 0.0
    with threadpool_limits(limits=cores):
        for n in w.prefill_nodes:
            q = host64(gpu["q_pre"][n])
            K, V = path_kv(n)
            got = host64(gpu["o_pre"][n])
            start = w.node_start(n)
            rows = sorted({int(x) for x in np.linspace(0, len(q) - 1, min(64, len(q)))})
            t0 = time.perf_counter()
            for j in rows:
                p = start + j
                want = A.extend(q[j:j + 1], K[:p + 1], V[:p + 1], p, w.sm_scale)
                hist["prefill"].add(got[j], want[0])
            dt_ = time.perf_counter() - t0
            t_pre_sampled += dt_
            t_pre += dt_ * len(q) / len(rows)
        t_ext = t_dec = 0.0
        n_req = 0
        for i in order:
            i = int(i)
            if n_req and t_pre_sampled + t_ext + t_dec >= budget:
                break
            K, V = context(i)
            P = len(w.prefix_tokens(reqs[i]))
            q = q_ext[starts[i]:starts[i + 1]]
            t0 = time.perf_counter()
            want = A.extend(q, K[:P + len(q)], V[:P + len(q)], P, w.sm_scale)
            t_ext += time.perf_counter() - t0
            hist["extend"].add(o_ext[starts[i]:starts[i + 1]], want)
            base = len(K) - T
            for t in steps:
                t0 = time.perf_counter()
                want = A.decode(q_dec[t, i], K[:base + t + 1], V[:base + t + 1], w.sm_scale)
                t_dec += time.perf_counter() - t0
                hist["decode"].add(o_dec[t][i], want)
            n_req += 1
    sampled = t_pre_sampled + t_ext + t_dec
    t_ext /= n_req
    t_dec /= len(steps) * n_req
    est = t_pre + B * t_ext + B * T * t_dec
    cpu = {"value": round(tokens_per_step / est, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"float64 numpy oracle on {cores} threads: up to 64 rows of each prefilled prefix, the extend "
                     f"of {n_req} of {B} requests and their decode at {len(steps)} of {T} steps; scaled to one "
                     f"step = {est:.3g} s",
           "sample_seconds": round(sampled, 2)}
    err = {k: v.report() for k, v in hist.items() if v.n}
    err["compared"] = "the last step's outputs (the last step with kernel timing) over the oracle's sample, element-wise"
    return cpu, err


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path is a single-GPU kernel library measured on one MI355X; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.ceilings:
        ceilings()
        return
    if args.page_size != 1 and args.workload != "classify_heavy":
        print("--page-size applies to the classify_heavy workload", file=sys.stderr)
        sys.exit(2)
    res = bench_classify_heavy(args) if args.workload == "classify_heavy" else bench_tree(args)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
