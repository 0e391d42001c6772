#!/usr/bin/env python3
"""Paged GQA attention on one MI355X: decode KV GB/s and us per call.

    python bench.py [--steps K] [--warmup W]            # the whole suite
    python bench.py --workload N [--page-size P]        # one workload

One step is one pass of the whole decode path over one batch of synthetic
input: the split pass (block-table gather, q.k, soft-cap/window mask, online
softmax, p.v, split partials with log-sum-exp) and the merge of the splits.
The headline workload is the Llama-3-8B-shaped decode (64 sequences, 32/8
heads, head_dim 128, bf16, page size 16, lengths uniform in [512, 4096]).
With no --workload the line also carries, under "workloads", the tiny decode,
the long-context decode at page sizes 64 and 1, the fp8-KV decode, a G = 1
(multi-head) decode and the prefix-prefill/extend workload, each with its
own time per call, roofline and CPU baseline.

Inputs are resident in HBM before timing starts; consecutive steps read
different copies of the inputs so no step finds the previous step's data in
the 256 MB last-level cache.  Prints one JSON line.

`--op verify` runs q_len query tokens per sequence on a decode workload,
`--op mla` the latent-cache decode (576/512 head dims), `--op append` the
KV-cache append, `--op mha` the G = 1 decode alone.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
MALL_BYTES = 256 << 20
METRIC = "paged-attn decode KV GB/s (fraction of HBM peak) + us/call on 1 MI355X"
# the sources each measured kernel is compiled from (counter figures taken
# from other sources are not reported)
DECODE_SPLIT_SOURCES = ["decode.hip", "decode_geom.h", "pa_device.h", "pa_internal.h"]
MLA_SPLIT_SOURCES = ["mla.hip", "decode_geom.h", "pa_device.h", "pa_internal.h"]
EXTEND_SOURCES = ["extend.hip", "pa_device.h", "pa_internal.h"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="one workload only (default: the suite, headline workload 2)")
    ap.add_argument("--page-size", type=int, default=None,
                    help="decode workloads: re-page the same tokens")
    ap.add_argument("--splits", type=int, default=0, help="force the split-pass block count")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU-baseline budget of the headline workload (0 disables the "
                         "oracle legs); the suite's other workloads take a third of it")
    ap.add_argument("--op", default="attention",
                    choices=["attention", "append", "verify", "mla", "mha"],
                    help="append: KV-cache append of the extend workload's new tokens; "
                         "verify: --q-len query tokens per sequence on a decode workload")
    ap.add_argument("--q-len", type=int, default=4,
                    help="query tokens per sequence for --op verify (1 + speculative tokens)")
    ap.add_argument("--mla-heads", type=int, default=16,
                    help="--op mla: query heads over the one latent kv head")
    ap.add_argument("--mla-batch", type=int, default=128, help="--op mla: sequences")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8_e4m3"],
                    help="cache element type for --op append")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_gqa_attention_02_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_record(kind: str, kernel: str, workload: str, srcs):
    """A committed rocprofv3 summary (profiles/<kernel>_<workload>.<kind>.json),
    if it was taken from the current kernel sources; else None."""
    safe = workload.replace("/", "-")
    path = os.path.join(ROOT, "profiles", f"{kernel}_{safe}.{kind}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != src_hash(*srcs):
        return None
    return rec


def traffic_for(kernel: str, workload: str, srcs):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary."""
    rec = profile_record("traffic", kernel, workload, srcs)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def cpu_baseline(run_once, alg_units, unit_scale, unit, budget_s, sample):
    """Time the oracle (as it stands) on the host cores, repeating the sample
    until the budget is used; returns the reported-baseline object."""
    import oracle
    threads = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        run_once(threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 3 * budget_s:
            break
    return {"value": alg_units * reps / el / unit_scale, "unit": unit, "cores": threads,
            "host_cpus": oracle.host_cpus(), "kind": "oracle",
            "sample": f"{sample}; {reps} pass(es) in {el:.1f} s"}


def copy_probe(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def time_steps(torch, step, K):
    """K back-to-back steps: wall-clock ms per step, and HIP-event ms per
    step on the stream the kernels are launched on (torch's current stream,
    which the binding passes to the library)."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for i in range(K):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return wall * 1e3 / K, e0.elapsed_time(e1) / K


def copies_for(kv_bytes: int) -> int:
    """Input copies so that consecutive steps never find their K/V in the
    last-level cache.  A workload of a few MB is launch-latency bound and
    cache resident whatever is done: one copy."""
    if kv_bytes < (8 << 20):
        return 1
    return max(2, math.ceil(2 * MALL_BYTES / kv_bytes) + 1)


def decode_entry(args, torch, pa, I, case, steps, warmup, cpu_s, seed_note):
    """One decode workload: whole-call time per step (wall clock and HIP
    events), the split kernel's time per launch (HIP events around K
    back-to-back launches on the kernels' stream), roofline and oracle."""
    dev = "cuda:0"
    latent = case.dv != case.head_dim
    alg = case.algorithmic_bytes()
    copies = copies_for(case.kv_bytes())
    tensors = [I.decode_tensors(case, dev) for _ in range(copies)]
    t0 = tensors[0]
    plan = pa.decode_plan(t0["q"], t0["k_pool"], t0["block_table"], case.max_kv_len,
                          window=case.window, num_splits=args.splits or case.num_splits,
                          head_dim_v=case.dv if latent else 0)
    out = torch.empty(case.batch, case.num_q_heads, case.dv, dtype=torch.bfloat16,
                      device=dev)
    ws = pa.workspace_for(plan, dev)

    def call(fn, i):
        t = tensors[i % copies]
        fn(plan, t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
           case.scale, softcap=case.softcap, window=case.window,
           k_scale=case.k_scale, v_scale=case.v_scale, out=out, workspace=ws)

    for i in range(warmup):
        call(pa.decode, i)
    ms_step, ev_ms = time_steps(torch, lambda i: call(pa.decode, i), steps)
    # the split pass (the kernel that streams the cache) alone: K launches
    # back to back, each on another copy of the inputs
    _, split_ms = time_steps(torch, lambda i: call(pa.decode_split, i), steps)
    torch.cuda.synchronize()
    kernel = "decode_split" if not latent else "mla_split"
    srcs = MLA_SPLIT_SOURCES if latent else DECODE_SPLIT_SOURCES
    achieved = alg / (split_ms * 1e-3) / 1e9
    trace = profile_record("trace", "decode_split", case.name, srcs)
    e = {
        "workload": f"{case.name} decode",
        "batch": case.batch, "num_q_heads": case.num_q_heads,
        "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim, "head_dim_v": case.dv,
        "page_size": case.page_size, "kv_dtype": case.kv_dtype, "window": case.window,
        "softcap": case.softcap, "total_tokens": int(case.seq_lens.sum()),
        "seed": seed_note, "input_copies": copies,
        "ms_per_step": ms_step,
        "us_per_call": ev_ms * 1e3,
        "value": alg / (ms_step * 1e-3) / 1e9, "unit": "GB/s",
        "hbm_frac": alg / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes": alg, "kv_bytes": case.kv_bytes(),
        "plan": plan.describe(),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_for("decode_split", case.name, srcs),
                     "us_per_launch": split_ms * 1e3,
                     "timing": f"HIP events around {steps} back-to-back split-pass launches",
                     # the committed rocprofv3 kernel average of these sources, and
                     # the fraction it gives
                     "rocprof_us_per_launch": None if trace is None else trace["avg_us"],
                     "frac_rocprof": None if trace is None else
                     alg / (trace["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS},
    }
    if cpu_s > 0:
        import oracle
        e["cpu_baseline"] = cpu_baseline(
            lambda th: oracle.decode(case, threads=th), alg, 1e9, "GB/s", cpu_s,
            f"the whole workload ({case.batch} sequences, {int(case.seq_lens.sum())} "
            f"tokens), fp64 oracle")
    del tensors
    return e


def extend_entry(args, torch, pa, I, steps, warmup, cpu_s):
    dev = "cuda:0"
    case = I.extend_config(5)
    flops = case.flops()
    t = I.extend_tensors(case, dev)
    plan = pa.extend_plan(t["q"], t["k_pool"], t["block_table"], case.batch,
                          case.max_kv_len, case.max_q_len, window=case.window,
                          num_splits=args.splits)
    out = torch.empty_like(t["q"])
    ws = pa.workspace_for(plan, dev)

    def step(i):
        pa.extend(plan, t["q"], t["k_new"], t["v_new"], t["cu_seqlens_q"], t["ctx_lens"],
                  t["k_pool"], t["v_pool"], t["block_table"], case.scale,
                  softcap=case.softcap, window=case.window, out=out, workspace=ws)

    for i in range(warmup):
        step(i)
    ms_step, k_ms = time_steps(torch, step, steps)
    achieved = flops / (k_ms * 1e-3) / 1e12
    trace = profile_record("trace", "extend", "extend", EXTEND_SOURCES)
    sq = profile_record("sq", "extend", "extend", EXTEND_SOURCES)
    traffic = traffic_for("extend", "extend", EXTEND_SOURCES)
    # bytes every call must move at least once: the attended context K/V,
    # the new K/V rows, Q and out
    D, Hq, Hkv = case.head_dim, case.num_q_heads, case.num_kv_heads
    # (with a window W the first new token, at position C, sees the context
    # keys from C - W + 1)
    ctx_keys = sum((min(int(c), case.window - 1) if case.window > 0 else int(c)) if n else 0
                   for c, n in zip(case.ctx_lens, case.q_lens))
    unique = (ctx_keys + case.total_q) * Hkv * D * 2 * 2 + 2 * case.total_q * Hq * D * 2
    e = {
        "workload": "extend", "batch": case.batch,
        "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
        "head_dim": case.head_dim, "page_size": case.kv.page_size,
        "total_q": case.total_q, "context_tokens": int(case.ctx_lens.sum()), "seed": 5,
        "ms_per_step": ms_step, "us_per_call": k_ms * 1e3,
        "value": flops / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s",
        "algorithmic_flops": flops, "unique_bytes": unique, "plan": plan.describe(),
        "roofline": {"bound": "mfma", "kernel": "extend (whole call: scan, blocks, merge)",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic,
                     "traffic_over_unique": None if traffic is None else traffic / unique,
                     "timing": f"HIP events around {steps} back-to-back calls",
                     # committed rocprofv3 averages of these sources: the main
                     # kernel, and the three kernels of a call together
                     "rocprof_us_per_launch": None if trace is None else trace["avg_us"],
                     "rocprof_us_per_call": None if trace is None else trace["call_us"],
                     "frac_rocprof": None if trace is None else
                     flops / (trace["call_us"] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "mfma_busy": None if sq is None else sq.get("mfma_busy")},
    }
    if cpu_s > 0:
        import numpy as np
        import oracle
        rng = np.random.default_rng(0)
        rows = np.sort(rng.choice(case.total_q, size=64, replace=False))
        pairs = 0
        cu, ctx = case.cu_seqlens_q, case.ctx_lens
        for r in rows:
            b = int(np.searchsorted(cu, r, side="right") - 1)
            pairs += int(ctx[b]) + int(r - cu[b]) + 1
        e["cpu_baseline"] = cpu_baseline(
            lambda th: oracle.extend(case, rows=rows, threads=th),
            4 * case.head_dim * case.num_q_heads * pairs, 1e12, "TFLOP/s", cpu_s,
            "64 seeded random rows of the workload, all heads")
    return e


def line(e, args, metric):
    """The one JSON line: an entry's figures at the top level."""
    config = {k: e[k] for k in ("workload", "batch", "num_q_heads", "num_kv_heads",
                                "head_dim", "head_dim_v", "page_size", "kv_dtype", "window",
                                "softcap", "total_tokens", "total_q", "context_tokens",
                                "seed", "input_copies") if k in e}
    kv = e.get("kv_dtype", "bf16")
    res = {"metric": metric, "value": e["value"], "unit": e["unit"], "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": e["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if kv == "bf16" else "fp8_e4m3 KV, bf16 Q/out",
           "data": "synthetic", "config": config}
    for k in ("us_per_call", "hbm_frac", "algorithmic_bytes", "algorithmic_flops", "kv_bytes",
              "unique_bytes", "plan", "roofline", "cpu_baseline"):
        if k in e:
            res[k] = e[k]
    return res


def suite(args, torch, pa, I):
    """The headline workload (Llama-3-8B-shaped decode) and, nested, every
    other workload with its own figures."""
    say = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    nested_cpu = args.cpu_seconds / 3
    say("llama3-8b decode")
    head = decode_entry(args, torch, pa, I, I.decode_config(2), args.steps, args.warmup,
                        args.cpu_seconds, 2)
    res = line(head, args, METRIC)
    w = {}
    few = max(5, args.steps // 2)
    plan = [("tiny", lambda: I.decode_config(1), 1),
            ("long-context P64", lambda: I.decode_config(3), 3),
            ("long-context P1", lambda: I.decode_config(3, page_size=1),
             "3 (tokens re-paged with seed 103)"),
            ("fp8-kv", lambda: I.decode_config(4), 4),
            ("mha G1", lambda: I.mha_config(), 7)]
    for name, make, seed in plan:
        say(name)
        w[name] = decode_entry(args, torch, pa, I, make(), few, max(2, args.warmup // 2),
                               nested_cpu, seed)
        torch.cuda.empty_cache()
    say("extend")
    w["extend"] = extend_entry(args, torch, pa, I, few, max(2, args.warmup // 2), nested_cpu)
    res["workloads"] = w
    return res


def bench_verify(args, torch, pa, I):
    """Speculative verify: a decode workload's batch with q_len query tokens
    per sequence (its last q_len cached tokens), one split pass and merge."""
    import numpy as np
    dev = "cuda:0"
    wl = args.workload or 2
    case = I.decode_config(wl, page_size=args.page_size)
    ql = args.q_len
    alg = case.verify_bytes(ql)
    copies = copies_for(case.kv_bytes())
    tensors = [I.decode_tensors(case, dev) for _ in range(copies)]
    rng = np.random.default_rng(1000 + wl)
    q = I._dev(I.bf16_bits(rng.standard_normal(
        (case.batch, ql, case.num_q_heads, case.head_dim), dtype=np.float32)), dev,
        torch.bfloat16)
    t0 = tensors[0]
    plan = pa.verify_plan(q, t0["k_pool"], t0["block_table"], case.max_kv_len,
                          window=case.window, num_splits=args.splits)
    out = torch.empty_like(q)
    ws = pa.workspace_for(plan, dev)

    def step(i):
        t = tensors[i % copies]
        pa.verify(plan, q, t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                  case.scale, softcap=case.softcap, window=case.window,
                  k_scale=case.k_scale, v_scale=case.v_scale, out=out, workspace=ws)

    for i in range(args.warmup):
        step(i)
    K = args.steps
    ms_step, ev_ms = time_steps(torch, step, K)
    achieved = alg / (ev_ms * 1e-3) / 1e9
    rows = ql * case.num_q_heads // case.num_kv_heads
    return {
        "metric": "paged-attn verify KV GB/s (fraction of HBM peak) + us/call on 1 MI355X",
        "value": alg / (ms_step * 1e-3) / 1e9, "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if case.kv_dtype == "bf16" else "fp8_e4m3 KV, bf16 Q/out",
        "data": "synthetic",
        "config": {"workload": f"{case.name} verify, q_len {ql}", "batch": case.batch,
                   "q_len": ql, "rows_per_kv_head": rows,
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "head_dim_v": case.dv,
                   "page_size": case.page_size,
                   "kv_dtype": case.kv_dtype, "window": case.window,
                   "softcap": case.softcap, "total_tokens": int(case.seq_lens.sum()),
                   "seed": wl, "input_copies": copies},
        "us_per_call": ev_ms * 1e3, "algorithmic_bytes": alg,
        "plan": plan.describe(),
        "roofline": {"bound": "hbm", "kernel": "decode_split + merge (whole call)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
    }


def bench_append(args, torch, pa, I):
    """The extend workload's new tokens (bf16 K/V rows) written into a paged
    cache at each sequence's next positions (one kernel per step)."""
    import numpy as np
    dev = "cuda:0"
    case = I.extend_config(5)
    T, Hkv, D, P = case.total_q, case.num_kv_heads, case.head_dim, 16
    lens = [int(c) + int(n) for c, n in zip(case.ctx_lens, case.q_lens)]
    rng = np.random.default_rng(5)
    table, num_pages = I.deal_pages(lens, P, rng)
    slots = np.concatenate([table[b, (int(c) + np.arange(int(n))) // P] * P +
                            (int(c) + np.arange(int(n))) % P
                            for b, (c, n) in enumerate(zip(case.ctx_lens, case.q_lens))])
    fp8 = args.kv_dtype == "fp8_e4m3"
    elem = 1 if fp8 else 2
    alg = T * Hkv * D * (2 + elem) * 2 + 8 * T
    copies = max(2, math.ceil(2 * MALL_BYTES / (T * Hkv * D * 2 * 2)) + 1)
    kv = [(torch.randn(T, Hkv, D, device=dev).to(torch.bfloat16),
           torch.randn(T, Hkv, D, device=dev).to(torch.bfloat16)) for _ in range(copies)]
    pdt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    k_pool = torch.zeros(num_pages, P, Hkv, D, dtype=pdt, device=dev)
    v_pool = torch.zeros_like(k_pool)
    st = torch.from_numpy(slots.astype(np.int64)).to(dev)
    ks, vs = (0.8, 1.3) if fp8 else (1.0, 1.0)

    def step(i):
        k, v = kv[i % copies]
        pa.cache_append(k, v, k_pool, v_pool, st, k_scale=ks, v_scale=vs)

    for i in range(args.warmup):
        step(i)
    K = args.steps
    ms_step, ev_ms = time_steps(torch, step, K)
    achieved = alg / (ev_ms * 1e-3) / 1e9
    return {
        "metric": "paged KV-cache append GB/s (fraction of HBM peak) on 1 MI355X",
        "value": alg / (ms_step * 1e-3) / 1e9, "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, " + ("fp8_e4m3" if fp8 else "bf16") + " cache", "data": "synthetic",
        "config": {"workload": "append of the extend workload's new tokens", "tokens": T,
                   "num_kv_heads": Hkv, "head_dim": D, "page_size": P,
                   "kv_dtype": args.kv_dtype, "input_copies": copies},
        "us_per_call": ev_ms * 1e3, "algorithmic_bytes": alg,
        "roofline": {"bound": "hbm", "kernel": "cache_append", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not "
              "supported (nothing is sharded across GPUs)", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import torch
    if args.copy_probe:
        copy_probe(torch)
        return
    import paged_gqa_attention_02_amd as pa
    from paged_gqa_attention_02_amd import inputs as I
    pa.lib()
    if args.op == "append":
        res = bench_append(args, torch, pa, I)
    elif args.op == "verify":
        if args.workload == 5:
            sys.exit("bench.py: --op verify runs on a decode workload (1-4)")
        res = bench_verify(args, torch, pa, I)
    elif args.op in ("mla", "mha"):
        case = (I.mla_config(args.mla_heads, args.mla_batch, args.page_size or 64)
                if args.op == "mla" else I.mha_config(args.page_size or 16))
        e = decode_entry(args, torch, pa, I, case, args.steps, args.warmup, args.cpu_seconds,
                         6 if args.op == "mla" else 7)
        res = line(e, args, METRIC)
    elif args.workload == 5:
        e = extend_entry(args, torch, pa, I, args.steps, args.warmup, args.cpu_seconds)
        res = line(e, args, "paged-attn extend TFLOP/s (fraction of MFMA bf16 peak) on 1 MI355X")
    elif args.workload is not None:
        e = decode_entry(args, torch, pa, I, I.decode_config(args.workload, args.page_size),
                         args.steps, args.warmup, args.cpu_seconds, args.workload)
        res = line(e, args, METRIC)
    else:
        res = suite(args, torch, pa, I)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
