"""Benchmark: one step = the whole hot path over one batch of a seeded
multi-turn-chat radix-tree workload on one MI355X.

Workload (default): GQA 32 q-heads / 8 kv-heads, head_dim 128, bf16; a cached
radix tree of depth 4 and branching 4 (340 segment nodes, 256 leaves) with
segment lengths uniform in [256, 1024]; pool slots handed out in a seeded
random order.  Each of the 256 leaf requests brings 128 new tokens and then
decodes 256 tokens.

A step, all of it inside the timed region:
  radix match + slot allocation + table rows (host C++)  -> upload rows
  KV scatter of the 32768 new tokens                      (HIP)
  extend attention, new tokens over prefix + themselves   (HIP, MFMA)
  commit: insert the prompts into the tree                (host C++)
  decode share plan from the tree                         (host C++) -> upload
  256 decode steps: KV scatter + split-K decode + merge   (HIP)
  release of the decode slots                             (host C++)
Every step brings fresh new tokens (the previous step's are cached by then),
so every step does the same work.  Inputs (q, k, v) are generated on the GPU
before timing and stay resident in HBM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM bytes per launch of the decode kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
# counters, with the sha256 of the kernel source they were taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attention_multi_turn_tree_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "prefix_shared_kv_amd", "csrc", "attention.hip")


def measured_traffic():
    """Counter-measured bytes per decode launch, or None when absent or taken
    on a different kernel source."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
        if kv.get("kernel_source_sha256") != src:
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
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--chunk", type=int, default=512, help="decode split size (positions per work item)")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=32, help="requests in the oracle sample")
    ap.add_argument("--cpu-decode-steps", type=int, default=32, help="decode steps per request in the oracle sample")
    ap.add_argument("--seed", type=int, default=4)
    ap.add_argument("--no-shuffle", action="store_true", help="hand out pool slots in order (no gather scatter)")
    ap.add_argument("--decode-rows", type=int, default=0, help="narrow decode by groups of four kv heads (rc_set_tuning)")
    ap.add_argument("--host-phases", action="store_true", help="report host wall time per phase of the last step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run kv_store into contiguous slots (a plain copy of known size) and print its bytes; "
                         "the scale for rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path is a single-GPU kernel library and this build runs on "
              "one MI355X; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    import prefix_shared_kv_amd as pk
    from prefix_shared_kv_amd.engine import Engine
    from synth import drive
    from synth import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pk.set_tuning("decode_rows", args.decode_rows)
    w = W.multi_turn_tree(seed=args.seed, n_decode=args.decode_steps)
    sh = w.shape
    B = len(w.requests)
    E = len(w.requests[0].ext_tokens)
    T = args.decode_steps
    n_steps_total = args.warmup + args.steps
    cached = sum(len(n.tokens) for n in w.nodes)
    pool = cached + n_steps_total * B * E + B * (E + T) + 1024
    kvs = pk.KVShape(sh.num_q_heads, sh.num_kv_heads, sh.head_dim, torch.bfloat16, pool)
    stride = max(len(w.prompt_tokens(r)) for r in w.requests) + T + 8
    order = None if args.no_shuffle else np.random.default_rng(args.seed).permutation(pool).astype(np.int32)
    eng = Engine(kvs, stride, B + 8, dev, free_order=order)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def randn(*s):
        return torch.randn(*s, device=dev, generator=gen, dtype=torch.float32).to(torch.bfloat16)

    # ---- cached tree (untimed set-up) ----
    for nid in drive.node_order(w):
        n = len(w.nodes[nid].tokens)
        eng.populate(drive.path_tokens(w, nid), randn(n, sh.num_kv_heads, sh.head_dim),
                     randn(n, sh.num_kv_heads, sh.head_dim), expect_cached=w.node_start(nid))
    log("cached tree populated")
    # ---- inputs resident in HBM ----
    q_ext = randn(B * E, sh.num_q_heads, sh.head_dim)
    k_ext = randn(B * E, sh.num_kv_heads, sh.head_dim)
    v_ext = randn(B * E, sh.num_kv_heads, sh.head_dim)
    q_dec = randn(T, B, sh.num_q_heads, sh.head_dim)
    k_dec = randn(T, B, sh.num_kv_heads, sh.head_dim)
    v_dec = randn(T, B, sh.num_kv_heads, sh.head_dim)
    o_ext = torch.empty_like(q_ext)
    o_dec = torch.empty(B, sh.num_q_heads, sh.head_dim, device=dev, dtype=torch.bfloat16)
    prefix = [w.prefix_tokens(r) for r in w.requests]

    def prompts(step):
        out = []
        for r, p in zip(w.requests, prefix):
            e = r.ext_tokens.copy()
            e[0] = (int(e[0]) + step) % W.VOCAB
            out.append(np.concatenate([p, e]))
        return out

    plan_info = {}

    phases = {}

    def one_step(step):
        tick = time.perf_counter()

        def mark(name):
            nonlocal tick
            now = time.perf_counter()
            phases[name] = round((now - tick) * 1e3, 3)
            tick = now

        toks = prompts(step)
        mark("prompts")
        b = eng.schedule(toks, reserve=T)
        mark("schedule")
        eng.extend(b, q_ext, k_ext, v_ext, w.sm_scale, o=o_ext)
        mark("extend_launch")
        eng.commit(b)
        mark("commit")
        st = eng.prepare_decode(b, [len(t) for t in toks], T, chunk=args.chunk)
        mark("prepare_decode")
        plan_info.update(st.plan.summary)
        for t in range(T):
            eng.decode_step(st, t, q_dec[t], k_dec[t], v_dec[t], w.sm_scale, o=o_dec)
        mark("decode_launches")
        eng.release(b)
        mark("release")
        return b

    for s in range(args.warmup):
        one_step(s)
    torch.cuda.synchronize()
    log(f"{args.warmup} warm-up steps done")
    pk.prof_collect()
    pk.prof_enable(True)
    t0 = time.perf_counter()
    for s in range(args.steps):
        b = one_step(args.warmup + s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = pk.prof_collect()
    pk.prof_enable(False)
    log(f"{args.steps} timed steps done: {elapsed / args.steps * 1e3:.2f} ms/step")

    # ---- algorithmic work per step ----
    D, Hq, Hkv = sh.head_dim, sh.num_q_heads, sh.num_kv_heads
    P = np.array([len(p) for p in prefix], np.float64)
    ext_flops = 4.0 * D * Hq * float(np.sum(E * P + E * (E + 1) / 2.0))
    row_bytes = 2 * Hkv * D * 2  # K and V, bf16, per position
    # unique positions read at decode step t: every cached node once, plus each request's own tokens
    own = E + np.arange(T) + 1  # new tokens + decode tokens so far (the current one included)
    uniq = cached + B * own
    # KV rows + slot index + q + o, and the current token's K/V: read once, written to its pool slot
    dec_bytes_steps = uniq * (row_bytes + 4) + 2 * B * Hq * D * 2 + 2 * B * row_bytes
    logical = B * (P.mean() + own)

    store_bytes = B * E * (2 * row_bytes + 4)  # the extend's new tokens: read K/V, write pool rows, slot index
    ext_name, mrg_name, st_name = "extend_bf16_d128", "decode_merge", "kv_store"
    dec_name = "decode_attention_d128"  # one launch per step: wide and narrow items
    ext_ms = prof[ext_name][1] / prof[ext_name][0]
    dec_ms = prof[dec_name][1] / prof[dec_name][0]
    mrg_ms = prof[mrg_name][1] / prof[mrg_name][0] if mrg_name in prof else 0.0  # merged in the decode kernel
    st_tot = prof[st_name][1] / args.steps
    ext_tflops = ext_flops / (ext_ms * 1e-3) / 1e12

    dec_gbs = float(np.mean(dec_bytes_steps)) / (dec_ms * 1e-3) / 1e9
    tokens_per_step = B * E + B * T
    ms_per_step = elapsed / args.steps * 1e3
    value = tokens_per_step * args.steps / elapsed

    res = {
        "metric": "extend-attn TFLOP/s (% MFMA peak) + decode-attn HBM GB/s, tokens/s, 1 GPU",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q/k/v N(0,1) drawn on the GPU)",
        "config": {
            "workload": "multi-turn chat radix tree: GQA 32/8, head_dim 128, bf16, depth 4 x branching 4 "
                        "(340 cached segments, 256 leaf requests), segments U[256,1024], 128 new tokens "
                        "per leaf then 256 decode steps, shuffled pool slots",
            "batch": B, "new_tokens_per_request": E, "decode_steps": T, "cached_tokens": cached,
            "mean_prefix": round(float(P.mean()), 1), "decode_chunk": args.chunk,
            "slot_order": "in order" if args.no_shuffle else "shuffled",
        },
        "roofline": {
            "bound": "hbm", "kernel": "decode_attn_bf16<128> (" + dec_name + ")",
            "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
            "avg_launch_ms": round(dec_ms, 5), "algorithmic_bytes_per_launch": float(np.mean(dec_bytes_steps)),
        },
        "extend": {
            "kernel": ext_name, "avg_launch_ms": round(ext_ms, 4), "algorithmic_tflop": round(ext_flops / 1e12, 4),
            "tflops": round(ext_tflops, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "frac": round(ext_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(B * E / (ext_ms * 1e-3), 1),
        },
        "decode": {
            "attention_ms": round(dec_ms, 5),
            "merge_avg_ms": round(mrg_ms, 5), "gbs": round(dec_gbs, 1),
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "unique_bytes_per_step": float(np.mean(dec_bytes_steps)),
            "logical_bytes_per_step": float(np.mean(logical) * row_bytes),
            "effective_gbs": round(float(np.mean(logical) * row_bytes) / (dec_ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(B / ((dec_ms + mrg_ms) * 1e-3), 1),
            "plan": {k: plan_info[k] for k in ("n_items", "shared_items", "max_splits")},
        },
        "kv_store": {"ms_per_step": round(st_tot, 4),
                     "gbs": round(store_bytes / (st_tot * 1e-3) / 1e9, 1)},
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in prof.items()},
    }
    if args.host_phases:
        res["host_phase_ms"] = phases
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample, args.cpu_decode_steps, tokens_per_step, T)
    print(json.dumps(res))


def cpu_baseline(w, n_req, n_dec, tokens_per_step, T):
    """The float64 oracle, as it stands, on a bounded sample of the same workload:
    the extend of `n_req` requests and their decode at `n_dec` evenly spaced steps;
    the per-request extend time and per-token decode time are scaled to one step."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    cores = len(os.sched_getaffinity(0))
    rids = list(range(n_req))
    steps = sorted({int(x) for x in np.linspace(0, T - 1, n_dec)})
    node_cache = {}

    def ctx(i):
        r = w.requests[i]
        for n in r.path:
            if n not in node_cache:
                node_cache[n] = w.node_kv(n)
        _, ek, ev = w.ext_qkv(i)
        return (np.concatenate([node_cache[n][0] for n in r.path] + [ek]),
                np.concatenate([node_cache[n][1] for n in r.path] + [ev]))

    inputs = {i: (w.ext_qkv(i)[0], *ctx(i)) for i in rids}
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for i in rids:
            q, K, V = inputs[i]
            A.extend(q, K, V, len(w.prefix_tokens(w.requests[i])), w.sm_scale)
        t_ext = (time.perf_counter() - t0) / n_req
        t_dec = 0.0
        for i in rids:
            _, K, V = inputs[i]
            for t in steps:
                extra = np.repeat(K[-1:], t + 1, axis=0)  # context length at step t; values do not matter for time
                Kt, Vt = np.concatenate([K, extra]), np.concatenate([V, extra])
                q = w.dec_qkv(i, t)[0]
                s = time.perf_counter()
                A.decode(q, Kt, Vt, w.sm_scale)
                t_dec += time.perf_counter() - s
        t_dec /= len(steps) * n_req
    B = len(w.requests)
    est_step = B * t_ext + B * T * t_dec
    return {"value": round(tokens_per_step / est_step, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 numpy oracle on {cores} threads: extend of {n_req} requests (128 new tokens over "
                      f"their cached prefix) and their decode at {len(steps)} steps spread over 0..{T - 1}; "
                      f"scaled to one step ({B} extends + {B}x{T} decode tokens) = {est_step:.0f} s",
            "sample_seconds": round(n_req * t_ext + len(steps) * n_req * t_dec, 2)}


if __name__ == "__main__":
    main()
