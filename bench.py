#!/usr/bin/env python3
"""Throughput of the fused Indexer-TopK on one MI355X.

Workload (default): the 1M-context prefill chunk -- 8,192 queries at the last
8,192 positions of L = 1,048,576 causal keys, H = 64 indexer heads, D = 128,
fp8 e4m3fn queries/keys with per-token fp32 scales, k = 2,048, sample = the
previous chunk's top-6,144 keys (computed untimed by running the previous
chunk through the same library).  Inputs are synthetic and seeded, resident in
device memory before timing starts.

One step = one litetopk_score_select call: sample pass, fused scan, finalize,
overflow fallback.  Metric: scored query-key pairs per second.  The line also
carries the roofline of the dominant kernel (the fused scan, timed with HIP
events on its stream), the unfused full-matrix baseline timed the same way,
bytes written per query, and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload prefill-1m-fp8]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# HBM-side bytes per launch of each scan kernel at its workload, from rocprofv3
# FETCH_SIZE / WRITE_SIZE scaled by a plain copy's readings (FETCH x2.0, WRITE
# x1.0; profiles/scan_kernel_prefill-1m-fp8.md, profiles/retr_scan_kernel_
# retrieval-8m-d768-bf16.md).  Valid only for the kernel sources with the
# recorded digest; reported as null otherwise.
KERNEL_SOURCES = ["device.hpp", "kernels_common.hpp", "internal.hpp", "indexer.hip"]
RETR_SOURCES = ["device.hpp", "kernels_common.hpp", "internal.hpp", "retrieve.hip"]
SCAN_TRAFFIC = {"digest": "2ccda14b383fdfde", "workload": "prefill-1m-fp8",
                "bytes": 2223930 * 1024 * 2.0 + 151690 * 1024 * 1.0}
RETR_TRAFFIC = {"digest": "cef33f8a64b052eb", "workload": "retrieval-8m-d768-bf16",
                "bytes": 8856324 * 1024 * 2.0 + 1293637 * 1024 * 1.0}

FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 matrix


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(inp, torch):
    dt = inp["dtype"]

    def raw(x):
        x = np.ascontiguousarray(x)
        if dt == "f32":
            return torch.from_numpy(x).cuda()
        if dt == "bf16":
            return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(x).cuda().view(torch.float8_e4m3fn)

    d = dict(q=raw(inp["q"]), k=raw(inp["k"]), w=torch.from_numpy(inp["w"]).cuda(),
             pos=torch.from_numpy(inp["pos"].astype(np.int32)).cuda(), q_scale=None, k_scale=None)
    if dt == "fp8":
        d["q_scale"] = torch.from_numpy(inp["q_scale"]).cuda()
        d["k_scale"] = torch.from_numpy(inp["k_scale"]).cuda()
    return d


def scan_source_digest(files=KERNEL_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "indexer_topk_long_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(inp, n_rows: int):
    """The CPU oracle, as it stands, on n_rows query rows spread over the chunk."""
    from oracle import oracle_indexer
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    T, L = inp["T"], inp["L"]
    rows = np.linspace(0, T - 1, n_rows).astype(np.int64)
    pairs = int(sum(min(int(inp["pos"][t]), L - 1) + 1 for t in rows))
    t0 = time.perf_counter()
    oracle_indexer(inp, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": pairs / dt, "unit": "pairs/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_rows} of {T} query rows (evenly spaced), all their causal keys: {pairs} pairs "
                      f"in {dt:.2f} s, fp64 numpy, including the fp64 decode of the keys"}


def bench_retrieval(args):
    """Separate line: the 8M x 768 bf16 retrieval workload (k = 1,024, random 3,072-row sample)."""
    import torch
    import indexer_topk_long_amd as ltk
    from workloads import retrieval_workload

    log("generating retrieval-8m-d768-bf16 on the GPU ...")
    r = retrieval_workload(args.workload, device="cuda")
    T, N, D, k = r["T"], r["N"], r["D"], r["topk"]
    q = torch.from_numpy(np.ascontiguousarray(r["q"]).view(np.int16)).cuda().view(torch.bfloat16)
    smp = torch.from_numpy(r["sample"]).cuda()
    ws = torch.empty(ltk.workspace_bytes(ltk.KIND_RETRIEVE, T, 1, D, N, k, len(r["sample"]), 1), dtype=torch.uint8,
                     device="cuda")
    for _ in range(args.warmup):
        ltk.retrieve(q, r["db"], k, sample=smp, workspace=ws)
    torch.cuda.synchronize()
    ev = ltk.HipEvents(args.steps)
    opts = [ltk.Opts(scan_event_start=a, scan_event_stop=b) for a, b in ev.pairs]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ltk.retrieve(q, r["db"], k, sample=smp, opts=opts[i], workspace=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    scan_ms = float(np.mean([ev.elapsed_ms(i) for i in range(args.steps)]))
    ev.close()
    _, st = ltk.retrieve(q, r["db"], k, sample=smp, workspace=ws, return_stats=True)
    pairs = T * N
    flops = 2.0 * D * pairs
    ach = flops / (scan_ms * 1e-3) / 1e12
    line = {"metric": "scored query-row pairs/s, retrieval k=1024", "value": pairs / (ms * 1e-3), "unit": "pairs/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded Gaussian-mixture database, random sample)",
            "config": {"workload": f"{args.workload}: T={T} queries, N={N} rows, D={D}, bf16, k={k}, "
                                   f"sample={len(r['sample'])} random rows", "pairs": pairs},
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                         "traffic": (RETR_TRAFFIC["bytes"] if scan_source_digest(RETR_SOURCES) == RETR_TRAFFIC["digest"]
                                     and args.workload == RETR_TRAFFIC["workload"] else None),
                         "kernel": "retr_scan_kernel", "kernel_ms": round(scan_ms, 4),
                         "db_read_GBps_at_kernel_time": round(N * D * 2 / (scan_ms * 1e-3) / 1e9, 1)},
            "candidates_per_query": round(st.cand_written / T, 1), "max_candidates": st.max_cand_per_query,
            "overflow_rows": st.overflow_rows, "cpu_baseline": None}
    print(json.dumps(line), flush=True)


def bench_prefill_chunks(args):
    """Separate line: a chunked prefill over the 1M-context keys (8,192-query chunks from
    position 0, each chunk's sample carried from the previous chunk's result)."""
    import torch
    import indexer_topk_long_amd as ltk
    from workloads import WORKLOADS, indexer_workload, prefill_queries

    name = "prefill-1m-fp8"
    c = WORKLOADS[name]
    log(f"generating the keys of {name} ...")
    inp = indexer_workload(name)
    k = torch.from_numpy(inp["k"]).cuda().view(torch.float8_e4m3fn)
    ks = torch.from_numpy(inp["k_scale"]).cuda()
    chunk = c["T"]
    nq = min(c["L"], args.prefill_chunks * chunk) if args.prefill_chunks > 0 else c["L"]
    qf = prefill_queries(name, device="cuda")
    ltk.prefill_chunked(qf, k, c["topk"], min(nq, 2 * chunk), chunk=chunk, n_sample=c["n_sample"], k_scale=ks)  # warmup
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = ltk.prefill_chunked(qf, k, c["topk"], nq, chunk=chunk, n_sample=c["n_sample"], k_scale=ks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ch = res["chunks"]
    pairs = sum(r["pairs"] for r in ch)
    hits = [r["sample_hit_rate"] for r in ch if r["sample_hit_rate"] is not None]
    sel_ms = sum(r["ms"] for r in ch)
    line = {"metric": "scored query-key pairs/s over a chunked prefill", "value": pairs / wall, "unit": "pairs/s",
            "n_gpus": 1, "steps": 1, "warmup": 1, "ms_per_step": round(wall * 1e3, 2), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
            "data": "synthetic (keys of prefill-1m-fp8; queries drawn on the device per chunk)",
            "config": {"workload": f"{name} keys, {len(ch)} chunks of {chunk} queries from position 0, "
                                   f"k={c['topk']}, sample = previous chunk's top-{c['n_sample']}",
                       "queries": nq, "pairs": pairs},
            "select_ms_total": round(sel_ms, 2),
            "workspace_bytes": res["workspace_bytes"],
            "candidates_per_query": {"first": round(ch[0]["candidates_per_query"], 1),
                                     "last": round(ch[-1]["candidates_per_query"], 1),
                                     "max_over_chunks": round(max(r["candidates_per_query"] for r in ch), 1)},
            "overflow_rows": sum(r["overflow_rows"] for r in ch),
            "sample_hit_rate": {"mean": round(float(np.mean(hits)), 4) if hits else None,
                                "min": round(float(np.min(hits)), 4) if hits else None,
                                "last": round(hits[-1], 4) if hits else None},
            "chunk_ms": {"first": round(ch[0]["ms"], 3), "last": round(ch[-1]["ms"], 3)}}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill-1m-fp8", help="indexer workload name (default: the 1M-context chunk)")
    ap.add_argument("--unfused-steps", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=72)
    ap.add_argument("--prefill-chunks", type=int, default=-1,
                    help="time a chunked prefill over the 1M-context keys: the first N chunks (0 = all 128)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        n = args.copy_probe // 4
        src = torch.arange(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {4 * n} bytes x 3")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import indexer_topk_long_amd as ltk
    from workloads import WORKLOADS, indexer_workload

    cfg = WORKLOADS[args.workload]
    if args.prefill_chunks >= 0:
        return bench_prefill_chunks(args)
    if cfg["kind"] == "retrieval":
        return bench_retrieval(args)
    log(f"generating workload {args.workload} ...")
    t0 = time.perf_counter()
    inp = indexer_workload(args.workload, with_prev=True)
    log(f"  generated in {time.perf_counter() - t0:.1f} s")
    T, L, H, D, k = inp["T"], inp["L"], inp["H"], inp["D"], inp["topk"]
    d = to_dev(inp, torch)
    prev = dict(inp["prev"])
    prev.update(k=inp["k"], k_scale=inp["k_scale"])
    pd = to_dev(prev, torch)
    n_sample = cfg["n_sample"]

    # previous chunk (bootstrapped with a seeded random sample), then its top-3k
    boot = torch.from_numpy(prev["sample"]).cuda()
    prev_idx = ltk.score_select(pd["q"], pd["k"], pd["w"], pd["pos"], k, sample=boot, q_scale=pd["q_scale"],
                                k_scale=pd["k_scale"])
    sample = ltk.next_sample(prev_idx, L, n_sample)
    del pd, prev_idx
    torch.cuda.synchronize()
    log("  previous-chunk sample ready")

    ws_bytes = ltk.workspace_bytes(ltk.KIND_SCORE_SELECT, T, H, D, L, k, n_sample, {"f32": 0, "bf16": 1, "fp8": 2}[inp["dtype"]])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def step(opts=None, **kw):
        return ltk.score_select(d["q"], d["k"], d["w"], d["pos"], k, sample=sample, q_scale=d["q_scale"],
                                k_scale=d["k_scale"], opts=opts, workspace=ws, **kw)

    for _ in range(args.warmup):
        ref = step()
    torch.cuda.synchronize()
    ev = ltk.HipEvents(args.steps)
    opts = [ltk.Opts(scan_event_start=a, scan_event_stop=b) for a, b in ev.pairs]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        out = step(opts[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    scan_ms = float(np.mean([ev.elapsed_ms(i) for i in range(args.steps)]))
    ev.close()
    log(f"  fused: {ms_step:.3f} ms/step, scan kernel {scan_ms:.3f} ms")

    pos = inp["pos"].astype(np.int64)
    pairs = int(np.sum(np.minimum(pos, L - 1) + 1))
    flops = 2.0 * H * D * pairs
    peak = {"fp8": FP8_PEAK_TFLOPS, "bf16": BF16_PEAK_TFLOPS, "f32": FP32_PEAK_TFLOPS}[inp["dtype"]]
    achieved = flops / (scan_ms * 1e-3) / 1e12

    _, st = step(return_stats=True)
    cands = st.cand_written / T
    bytes_q = (8.0 * st.cand_written + 4.0 * T * k) / T
    full_q = 4.0 * L

    # unfused baseline (full fp32 score matrix + radix select), same inputs
    unf = None
    if args.unfused_steps > 0:
        uws = torch.empty((T * L * 4), dtype=torch.uint8, device="cuda")
        uout = ltk.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"],
                                        k_scale=d["k_scale"], workspace=uws)
        torch.cuda.synchronize()
        same = bool(torch.equal(torch.sort(uout, dim=1).values, torch.sort(out, dim=1).values))
        t0 = time.perf_counter()
        for _ in range(args.unfused_steps):
            ltk.unfused_score_select(d["q"], d["k"], d["w"], d["pos"], k, q_scale=d["q_scale"],
                                     k_scale=d["k_scale"], workspace=uws)
        torch.cuda.synchronize()
        ums = (time.perf_counter() - t0) * 1e3 / args.unfused_steps
        unf = {"ms_per_step": round(ums, 3), "value": pairs / (ums * 1e-3), "unit": "pairs/s",
               "bytes_written_per_query": 4.0 * L + 4.0 * k, "same_index_sets_as_fused": same}
        del uws
        log(f"  unfused: {ums:.3f} ms/step, same sets: {same}")
    consistent = bool(torch.equal(torch.sort(out, dim=1).values, torch.sort(ref, dim=1).values))

    cpu = None
    if not args.no_cpu_baseline:
        log("  timing the CPU oracle ...")
        cpu = cpu_baseline(inp, args.cpu_rows)

    line = {
        "metric": "scored query-key pairs/s at 1M context, k=2048",
        "value": pairs / (ms_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp["dtype"],
        "data": "synthetic (seeded concentrated-score generator; previous-chunk sample)",
        "config": {"workload": f"{args.workload}: T={T} queries at positions {int(pos[0])}..{int(pos[-1])}, "
                               f"L={L} causal keys, H={H}, D={D}, {inp['dtype']}, k={k}, "
                               f"sample=previous chunk top-{n_sample}",
                   "T": T, "L": L, "H": H, "D": D, "topk": k, "n_sample": n_sample, "pairs": pairs},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": (SCAN_TRAFFIC["bytes"] if scan_source_digest() == SCAN_TRAFFIC["digest"]
                                 and args.workload == SCAN_TRAFFIC["workload"] else None),
                     "kernel": "scan_kernel (fused score + filter)", "kernel_ms": round(scan_ms, 4),
                     "algorithmic_flops_per_launch": flops},
        "bytes_written_per_query": round(bytes_q, 1),
        "full_matrix_bytes_per_query": full_q,
        "candidates_per_query": round(cands, 1),
        "overflow_rows": st.overflow_rows,
        "repeat_consistent": consistent,
        "unfused_baseline": unf,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
