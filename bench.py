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

# HBM-side bytes per launch of each measured kernel at its workload, from
# rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a plain copy's readings (FETCH
# x2.0, WRITE x1.0; profiles/scan_kernel_prefill-1m-fp8.md,
# profiles/retr_scan_kernel_retrieval-8m-d768-bf16.md,
# profiles/decode_step_decode-1m-fp8.md, profiles/dsa_pack_dsa-1m-fp8.md).
# Valid only for the kernel sources with the recorded digest; null otherwise.
KERNEL_SOURCES = ["device.hpp", "kernels_common.hpp", "internal.hpp", "indexer.hip"]
RETR_SOURCES = ["device.hpp", "kernels_common.hpp", "internal.hpp", "retrieve.hip"]
DSA_SOURCES = ["device.hpp", "internal.hpp", "dsa.hip"]
SCAN_TRAFFIC = {"digest": "a2b5049f774f6b45", "workload": "prefill-1m-fp8",
                "bytes": 2228843 * 1024 * 2.0 + 152471 * 1024 * 1.0}
RETR_TRAFFIC = {"digest": "ddb385e3e0aa1fa1", "workload": "retrieval-8m-d768-bf16",
                "bytes": 8615774 * 1024 * 2.0 + 1730362 * 1024 * 1.0}
DECODE_TRAFFIC = {"digest": "a2b5049f774f6b45", "workload": "decode-1m-fp8",
                  "bytes": 67674 * 1024 * 2.0 + 46 * 1024 * 1.0}
DSA_TRAFFIC = {"digest": "712d6bd147e58a78", "workload": "dsa-1m-fp8",
               "pack_bytes": 33067 * 1024 * 2.0 + 134174 * 1024 * 1.0,
               "gather_bytes": 744743 * 1024 * 2.0 + 2708540 * 1024 * 1.0}

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
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


def _retrieval_run(ltk, torch, q, db, k, smp, steps, warmup):
    """Timed retrieve calls: (ms per step, scan ms from HIP events, stats)."""
    T, D = q.shape
    N = db.shape[0]
    ws = torch.empty(ltk.workspace_bytes(ltk.KIND_RETRIEVE, T, 1, D, N, k, smp.numel(), 1), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup):
        ltk.retrieve(q, db, k, sample=smp, workspace=ws)
    torch.cuda.synchronize()
    ev = ltk.HipEvents(steps)
    opts = [ltk.Opts(scan_event_start=a, scan_event_stop=b) for a, b in ev.pairs]
    t0 = time.perf_counter()
    for i in range(steps):
        ltk.retrieve(q, db, k, sample=smp, opts=opts[i], workspace=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    scan_ms = float(np.mean([ev.elapsed_ms(i) for i in range(steps)]))
    ev.close()
    _, st = ltk.retrieve(q, db, k, sample=smp, workspace=ws, return_stats=True)
    return ms, scan_ms, st


def retrieval_cpu_baseline(r, db, topk: int, n_rows: int = 256, n_db: int = 1 << 20):
    """The CPU oracle, as it stands, on n_rows evenly spaced queries against
    the first n_db database rows (copied to the host); the pairs/s rate
    extrapolates to the whole workload."""
    import torch
    from oracle import oracle_retrieval
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    T = r["T"]
    n_db = min(n_db, db.shape[0])
    rows = np.linspace(0, T - 1, n_rows).astype(np.int64)
    dbh = db[:n_db].view(torch.int16).cpu().numpy().view(np.uint16)
    qh = np.ascontiguousarray(r["q"][rows])
    t0 = time.perf_counter()
    oracle_retrieval(qh, dbh, topk)
    dt = time.perf_counter() - t0
    pairs = n_rows * n_db
    return {"value": pairs / dt, "unit": "pairs/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_rows} of {T} queries (evenly spaced) against the first {n_db} of {db.shape[0]} "
                      f"database rows: {pairs} pairs in {dt:.2f} s, fp64 numpy including the fp64 decode; "
                      f"extrapolated to the workload"}


def bench_retrieval(args):
    """Separate line: the 8M x 768 bf16 retrieval workload (k = 1,024, random 3,072-row sample).

    With --retrieval-sweep K1,K2,...: one line over those k, each with a
    sample of 3k seeded-random rows, or with --sweep-sample earlier, the 3k
    rows an earlier batch's queries selected most often (that batch runs first
    on a random 3k sample; litetopk_next_sample ranks the rows)."""
    import torch
    import indexer_topk_long_amd as ltk
    from workloads import WORKLOADS, random_retrieval_sample_of, retrieval_queries, retrieval_workload

    log("generating retrieval-8m-d768-bf16 on the GPU ...")
    r = retrieval_workload(args.workload, device="cuda")
    T, N, D, k = r["T"], r["N"], r["D"], r["topk"]
    q = torch.from_numpy(np.ascontiguousarray(r["q"]).view(np.int16)).cuda().view(torch.bfloat16)

    def roofline(scan_ms, traffic):
        ach = 2.0 * D * T * N / (scan_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": "retr_scan_kernel",
                "kernel_ms": round(scan_ms, 4), "db_read_GBps_at_kernel_time": round(N * D * 2 / (scan_ms * 1e-3) / 1e9, 1)}

    if args.retrieval_sweep:
        c = WORKLOADS[args.workload]
        qp_raw, _ = retrieval_queries(T, D, c["n_centres"], c["sigma"], tag=c["tag"], batch=-1)
        qp = torch.from_numpy(np.ascontiguousarray(qp_raw).view(np.int16)).cuda().view(torch.bfloat16)
        rows = []
        for kk in [int(x) for x in args.retrieval_sweep.split(",")]:
            smp = torch.from_numpy(random_retrieval_sample_of(args.workload, 3 * kk)).cuda()
            if args.sweep_sample == "earlier":
                prev = ltk.retrieve(qp, r["db"], kk, sample=smp)
                smp = ltk.next_sample(prev, N, 3 * kk)
                del prev
            ms, scan_ms, st = _retrieval_run(ltk, torch, q, r["db"], kk, smp, args.steps, args.warmup)
            out = ltk.retrieve(q, r["db"], kk, sample=smp)
            hit = float(torch.isin(out, smp).float().mean().item())
            log(f"  k={kk}: {ms:.3f} ms/step, scan {scan_ms:.3f} ms, {st.cand_written / T:.0f} candidates/query")
            rows.append({"topk": kk, "ms_per_step": round(ms, 4), "value": T * N / (ms * 1e-3),
                         "roofline": roofline(scan_ms, None),
                         "candidates_per_query": round(st.cand_written / T, 1),
                         "max_candidates": st.max_cand_per_query, "overflow_rows": st.overflow_rows,
                         "sample_hit_rate": round(hit, 4)})
            del out, smp
        best = rows[-1]
        line = {"metric": "scored query-row pairs/s, retrieval k-sweep", "value": best["value"], "unit": "pairs/s",
                "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": best["ms_per_step"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded Gaussian-mixture database)",
                "config": {"workload": f"{args.workload}: T={T} queries, N={N} rows, D={D}, bf16, k in "
                                       f"{args.retrieval_sweep} (value and ms_per_step: the last k); sample = "
                                       + ("the 3k rows an earlier batch of queries selected most often"
                                          if args.sweep_sample == "earlier" else "3k seeded-random rows"),
                           "pairs": T * N},
                "roofline": best["roofline"], "sweep": rows, "cpu_baseline": None}
        if not args.no_cpu_baseline:
            log("  timing the CPU oracle ...")
            line["cpu_baseline"] = retrieval_cpu_baseline(r, r["db"], rows[-1]["topk"])
        print(json.dumps(line), flush=True)
        return

    smp = torch.from_numpy(r["sample"]).cuda()
    ms, scan_ms, st = _retrieval_run(ltk, torch, q, r["db"], k, smp, args.steps, args.warmup)
    pairs = T * N
    traffic = (RETR_TRAFFIC["bytes"] if scan_source_digest(RETR_SOURCES) == RETR_TRAFFIC["digest"]
               and args.workload == RETR_TRAFFIC["workload"] else None)
    line = {"metric": "scored query-row pairs/s, retrieval k=1024", "value": pairs / (ms * 1e-3), "unit": "pairs/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded Gaussian-mixture database, random sample)",
            "config": {"workload": f"{args.workload}: T={T} queries, N={N} rows, D={D}, bf16, k={k}, "
                                   f"sample={len(r['sample'])} random rows", "pairs": pairs},
            "roofline": roofline(scan_ms, traffic),
            "candidates_per_query": round(st.cand_written / T, 1), "max_candidates": st.max_cand_per_query,
            "overflow_rows": st.overflow_rows, "cpu_baseline": None}
    if args.unfused_steps > 0:
        # the unfused comparison path: the full T x N fp32 matrix, then a radix select per row
        log(f"  unfused retrieval ({T * N * 4 / 1e9:.1f} GB score matrix) ...")
        uws = torch.empty(ltk.workspace_bytes(ltk.KIND_UNFUSED_RETRIEVE, T, 1, D, N, k, 0, 1), dtype=torch.uint8,
                          device="cuda")
        uout = ltk.unfused_retrieve(q, r["db"], k, workspace=uws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.unfused_steps):
            ltk.unfused_retrieve(q, r["db"], k, workspace=uws)
        torch.cuda.synchronize()
        ums = (time.perf_counter() - t0) * 1e3 / args.unfused_steps
        fout = ltk.retrieve(q, r["db"], k, sample=smp)
        same = bool(torch.equal(torch.sort(uout, dim=1).values, torch.sort(fout, dim=1).values))
        line["unfused_baseline"] = {"ms_per_step": round(ums, 3), "value": pairs / (ums * 1e-3), "unit": "pairs/s",
                                    "speedup_of_fused": round(ums / ms, 2), "bytes_written": T * N * 4 + T * k * 4,
                                    "same_index_sets_as_fused": same}
        log(f"  unfused: {ums:.3f} ms/step ({ums / ms:.2f}x the fused step), same sets: {same}")
        del uws, uout, fout
    if not args.no_cpu_baseline:
        log("  timing the CPU oracle ...")
        line["cpu_baseline"] = retrieval_cpu_baseline(r, r["db"], k)
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
    # every query resident in device memory before the timed pass (8.6 GB at 1M)
    qf = prefill_queries(name, device="cuda")
    parts = [qf(c0, min(nq, c0 + chunk)) for c0 in range(0, nq, chunk)]
    q_all = torch.cat([p[0] for p in parts])
    w_all = torch.cat([p[1] for p in parts])
    qs_all = torch.cat([p[2] for p in parts]) if parts[0][2] is not None else None
    del parts
    queries = (q_all, w_all, qs_all)
    log(f"  {nq} queries resident ({q_all.numel() * q_all.element_size() / 2**30:.1f} GiB)")
    ltk.prefill_chunked(queries, k, c["topk"], min(nq, 2 * chunk), chunk=chunk, n_sample=c["n_sample"],
                        k_scale=ks, diagnostics=False)  # warmup
    torch.cuda.synchronize()
    # timed: the chunks enqueued back to back (no per-chunk host synchronisation)
    t0 = time.perf_counter()
    timed = ltk.prefill_chunked(queries, k, c["topk"], nq, chunk=chunk, n_sample=c["n_sample"], k_scale=ks,
                                diagnostics=False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pairs = sum(r["pairs"] for r in timed["chunks"])
    # untimed: the same pass again with per-chunk events and statistics
    res = ltk.prefill_chunked(queries, k, c["topk"], nq, chunk=chunk, n_sample=c["n_sample"], k_scale=ks)
    ch = res["chunks"]
    assert sum(r["pairs"] for r in ch) == pairs
    assert torch.equal(torch.sort(timed["last"], dim=1).values, torch.sort(res["last"], dim=1).values), \
        "timed and diagnostic passes selected different keys"
    hits = [r["sample_hit_rate"] for r in ch if r["sample_hit_rate"] is not None]
    sel_ms = sum(r["ms"] for r in ch)
    line = {"metric": "scored query-key pairs/s over a chunked prefill", "value": pairs / wall, "unit": "pairs/s",
            "n_gpus": 1, "steps": 1, "warmup": 1, "ms_per_step": round(wall * 1e3, 2), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
            "data": "synthetic (keys of prefill-1m-fp8; all queries drawn on the device before the timed pass)",
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


def bench_decode(args):
    """Separate line: decode steps over the 1M-context keys.

    A step scores T queries at the newest positions (T = 1: one new token;
    T = 8: a new token and seven draft tokens verified together) against every
    causal key and returns their exact top-k.  Its sample is the union of the
    last three steps' results (the decode counterpart of reusing the previous
    chunk's top-3k; duplicates are dropped on the device).  Steps advance by T
    positions.  Timed eagerly (one library call per step) and as one HIP graph
    of the same steps, whose results must hold the same index sets.
    """
    import torch
    import indexer_topk_long_amd as ltk
    from workloads import WORKLOADS, indexer_keys, prefill_queries, random_sample

    cfg = WORKLOADS[args.workload]
    base = cfg["keys"]
    c = WORKLOADS[base]
    T, L, H, D, k = cfg["T"], c["L"], c["H"], c["D"], c["topk"]
    log(f"generating the keys of {base} ...")
    kr, ksr = indexer_keys(base)
    kk = torch.from_numpy(kr).cuda().view(torch.float8_e4m3fn)
    ks = torch.from_numpy(ksr).cuda()
    del kr, ksr
    nw, n = args.warmup, args.steps
    total = 1 + nw + n                     # bootstrap, warmup, timed
    P0 = L - total * T
    qf = prefill_queries(base, device="cuda")
    steps = []
    for j in range(total):
        q, w, qs = qf(P0 + j * T, P0 + (j + 1) * T)
        steps.append((q, w, qs, torch.arange(P0 + j * T, P0 + (j + 1) * T, dtype=torch.int32, device="cuda")))
    n_boot = c["n_sample"]
    ws = torch.empty(ltk.workspace_bytes(ltk.KIND_SCORE_SELECT, T, H, D, L, k, max(3 * T * k, n_boot), 2),
                     dtype=torch.uint8, device="cuda")
    # the last three results live in one ring [3, T, k]: step j writes slot j % 3
    # and samples the whole ring (the call consumes its sample before it writes)
    ring = torch.empty((3, T, k), dtype=torch.int32, device="cuda")

    def step(j, sample, out, opts=None, **kw):
        q, w, qs, pos = steps[j]
        return ltk.score_select(q, kk, w, pos, k, sample=sample.reshape(-1), q_scale=qs, k_scale=ks, opts=opts,
                                workspace=ws, out=out, **kw)

    def run(j0, count, opts=None, keep=True):
        outs = []
        for i in range(count):
            j = j0 + i
            o = step(j, ring, ring[j % 3], opts[i] if opts else None)
            if keep:
                outs.append(o.clone())
        return outs

    # bootstrap step on a seeded random sample of the visible keys fills every
    # slot of the ring, then warmup
    boot = torch.from_numpy(random_sample(n_boot, P0, tag=c["tag"])).cuda()
    first = step(0, boot, None)
    ring.copy_(first.unsqueeze(0).expand(3, T, k))
    run(1, nw, keep=False)
    ring0 = ring.clone()
    torch.cuda.synchronize()
    ev = ltk.HipEvents(n)
    opts = [ltk.Opts(scan_event_start=a, scan_event_stop=b) for a, b in ev.pairs]
    t0 = time.perf_counter()
    for i in range(n):
        step(1 + nw + i, ring, ring[(1 + nw + i) % 3], opts[i])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / n
    scan_ms = float(np.mean([ev.elapsed_ms(i) for i in range(n)]))
    ev.close()
    ring_eager = ring.clone()
    log(f"  eager: {eager_ms * 1e3:.1f} us/step, scan kernel {scan_ms * 1e3:.1f} us")

    # the results of every timed step, kept step by step (untimed), for the checks
    ring.copy_(ring0)
    eager = run(1 + nw, n)
    torch.cuda.synchronize()

    def same_sets(a, b):
        return all(torch.equal(torch.sort(x, dim=1).values, torch.sort(y, dim=1).values) for x, y in zip(a, b))

    # the same n steps captured as one graph (it starts from the ring the timed steps started from)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ring.copy_(ring0)
        run(1 + nw, n, keep=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run(1 + nw, n, keep=False)
    ring.copy_(ring0)
    g.replay()
    torch.cuda.synchronize()
    graph_same = same_sets(ring, ring_eager)
    reps = 5
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()   # each replay continues from the ring the previous one left (steps of the same positions)
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / (reps * n)
    log(f"  graph: {graph_ms * 1e3:.1f} us/step, same as eager: {graph_same}")

    # figures of the last timed step
    jl = nw + n
    allh = [ring0[(1 + nw + i) % 3] for i in range(-3, 0)] + eager   # results, oldest first
    _, st = step(jl, torch.stack(allh[-4:-1]), torch.empty((T, k), dtype=torch.int32, device="cuda"),
                 return_stats=True)
    pos_last = steps[jl][3].cpu().numpy().astype(np.int64)
    pairs = int(np.sum(pos_last + 1))
    visible = int(pos_last.max()) + 1
    scan_bytes = visible * (D + 4) + T * H * D + T * H * 4 + T * 4
    hits = [float(torch.isin(allh[i], torch.cat([h.reshape(-1) for h in allh[i - 3:i]])).float().mean())
            for i in range(3, len(allh))]
    uout = ltk.unfused_score_select(steps[jl][0], kk, steps[jl][1], steps[jl][3], k, q_scale=steps[jl][2],
                                    k_scale=ks)
    same_unfused = same_sets([uout], [eager[-1]])
    del uout
    oracle = None
    if not args.no_cpu_baseline:
        log("  oracle on the last step's rows ...")
        from oracle import oracle_indexer
        q, w, qs, pos = steps[jl]
        inp = dict(kind="indexer", T=T, L=L, H=H, D=D, dtype="fp8", topk=k, q=q.view(torch.uint8).cpu().numpy(),
                   k=kk.view(torch.uint8).cpu().numpy(), q_scale=qs.cpu().numpy(), k_scale=ks.cpu().numpy(),
                   w=w.cpu().numpy(), pos=pos.cpu().numpy())
        t0 = time.perf_counter()
        ref_idx, _ = oracle_indexer(inp, rows=np.arange(T))
        dt = time.perf_counter() - t0
        got = eager[-1].cpu().numpy()
        overlap = float(np.mean([len(set(got[t].tolist()) & set(ref_idx[t].tolist())) / k for t in range(T)]))
        oracle = {"value": pairs / dt, "unit": "pairs/s", "cores": _cores(), "kind": "oracle",
                  "sample": f"the {T} query row(s) of the last decode step, all causal keys: {pairs} pairs in "
                            f"{dt:.2f} s, fp64 numpy",
                  "set_overlap_with_gpu": round(overlap, 6)}
    value = pairs / (graph_ms * 1e-3)
    line = {"metric": "scored query-key pairs/s per decode step at 1M context, k=2048", "value": value,
            "unit": "pairs/s", "n_gpus": 1, "steps": n, "warmup": nw, "ms_per_step": round(graph_ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
            "data": "synthetic (keys of prefill-1m-fp8; queries drawn on the device per step)",
            "config": {"workload": f"{args.workload}: {T} quer{'y' if T == 1 else 'ies'} per step, timed steps at "
                                   f"positions {P0 + (1 + nw) * T}..{L - 1}, L={L} keys, H={H}, D={D}, fp8, k={k}, "
                                   f"sample = union of the last 3 steps' results",
                       "T": T, "L": L, "H": H, "D": D, "topk": k},
            "tokens_per_s": T / (graph_ms * 1e-3),
            "launch": {"graph_us_per_step": round(graph_ms * 1e3, 2), "eager_us_per_step": round(eager_ms * 1e3, 2),
                       "graph_same_sets_as_eager": graph_same},
            "roofline": {"bound": "hbm", "achieved": round(scan_bytes / (scan_ms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(scan_bytes / (scan_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "traffic": (DECODE_TRAFFIC["bytes"] if scan_source_digest() == DECODE_TRAFFIC["digest"]
                                     and args.workload == DECODE_TRAFFIC["workload"] else None),
                         "kernel": "scan_kernel (fused score + filter)", "kernel_us": round(scan_ms * 1e3, 2),
                         "algorithmic_bytes_per_launch": scan_bytes},
            "candidates_per_query": round(st.cand_written / T, 1), "max_candidates": st.max_cand_per_query,
            "overflow_rows": st.overflow_rows,
            "sample_hit_rate": round(float(np.mean(hits)), 4) if hits else None,
            "same_index_sets_as_unfused": same_unfused,
            "cpu_baseline": oracle}
    print(json.dumps(line), flush=True)


def bench_dsa(args):
    """Separate line: LiteDSA packing of the 1M-context prefill chunk.

    The chunk's selections come from the library itself: the last two chunks
    of the 1M prefill run through prefill_chunked (the second samples the
    first's top-3k), and the last chunk's [8192, 2048] result is packed in
    groups of neighbouring queries.  Timed: litetopk_dsa_pack over the chunk
    and litetopk_dsa_gather of the shared key/value rows (synthetic bf16
    rows of the workload's width).
    """
    import torch
    import indexer_topk_long_amd as ltk
    from workloads import WORKLOADS, indexer_keys, prefill_queries

    cfg = WORKLOADS[args.workload]
    base = cfg["keys"]
    c = WORKLOADS[base]
    T, L, k, G, rb = c["T"], c["L"], c["topk"], cfg["group"], cfg["kv_row_bytes"]
    log(f"generating the keys of {base} ...")
    kr, ksr = indexer_keys(base)
    kk = torch.from_numpy(kr).cuda().view(torch.float8_e4m3fn)
    ks = torch.from_numpy(ksr).cuda()
    del kr, ksr
    qf = prefill_queries(base, device="cuda")
    first = L - 2 * T
    res = ltk.prefill_chunked(lambda c0, c1: qf(first + c0, first + c1), kk, k, 2 * T, chunk=T,
                              n_sample=c["n_sample"], k_scale=ks, first_pos=first, keep_outputs=True)
    idx = res["outputs"][-1].contiguous()
    del kk, ks, res
    torch.cuda.synchronize()
    log("  selections of the chunk ready")
    kv = torch.randint(-2 ** 15, 2 ** 15 - 1, (L, rb // 2), dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ng = T // G
    out = torch.empty((ng, G * k, rb // 2), dtype=torch.bfloat16, device="cuda")
    for _ in range(args.warmup):
        sh, m, n = ltk.dsa_pack(idx, L, G)
        ltk.dsa_gather(kv, sh, n, out=out)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    pack_ms, gather_ms = [], []
    for _ in range(args.steps):
        ev[0].record()
        sh, m, n = ltk.dsa_pack(idx, L, G)
        ev[1].record()
        ltk.dsa_gather(kv, sh, n, out=out)
        ev[2].record()
        ev[2].synchronize()
        pack_ms.append(ev[0].elapsed_time(ev[1]))
        gather_ms.append(ev[1].elapsed_time(ev[2]))
    pack_ms, gather_ms = float(np.mean(pack_ms)), float(np.mean(gather_ms))
    lens = n.cpu().numpy().astype(np.int64)
    valid = int((idx >= 0).sum().item())
    shared_rows = int(lens.sum())
    # the pack reads the selections and writes the lists, masks and lengths
    pack_bytes = T * k * 4 + 2 * ng * G * k * 4 + ng * 4
    gather_bytes = shared_rows * rb * 2 + shared_rows * 4
    log(f"  pack {pack_ms * 1e3:.1f} us, gather {gather_ms * 1e3:.1f} us, rows {valid} -> {shared_rows}")
    dsa_ok = scan_source_digest(DSA_SOURCES) == DSA_TRAFFIC["digest"] and args.workload == DSA_TRAFFIC["workload"]
    line = {"metric": "LiteDSA: selected query-key entries packed per second (1M-context chunk, k=2048)",
            "value": valid / (pack_ms * 1e-3), "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(pack_ms + gather_ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "int32",
            "data": "synthetic (the library's own selections for the prefill-1m-fp8 chunk; random key/value rows)",
            "config": {"workload": f"{args.workload}: the {T} selections (k={k}) of the last 1M-context chunk in "
                                   f"groups of {G} neighbouring queries; key/value rows of {rb} bytes",
                       "T": T, "topk": k, "group": G, "kv_row_bytes": rb},
            "pack_ms": round(pack_ms, 4), "gather_ms": round(gather_ms, 4),
            "shared_list": {"mean_len": round(float(lens.mean()), 1), "max_len": int(lens.max()),
                            "capacity": G * k, "compression": round(valid / shared_rows, 3)},
            "kv_bytes_per_query": {"own_lists": round(valid * rb / T, 1), "shared": round(shared_rows * rb / T, 1)},
            "roofline": {"bound": "hbm", "achieved": round(pack_bytes / (pack_ms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(pack_bytes / (pack_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "traffic": DSA_TRAFFIC["pack_bytes"] if dsa_ok else None,
                         "kernel": "dsa_pack_kernel", "algorithmic_bytes_per_launch": pack_bytes},
            "gather_roofline": {"bound": "hbm", "achieved": round(gather_bytes / (gather_ms * 1e-3) / 1e9, 1),
                                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                "frac": round(gather_bytes / (gather_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                "traffic": DSA_TRAFFIC["gather_bytes"] if dsa_ok else None,
                                "algorithmic_bytes_per_launch": gather_bytes},
            "cpu_baseline": None}
    print(json.dumps(line), flush=True)


def measure_peaks(torch, mfma_iters: int = 200, read_bytes: int = 4 << 30) -> dict:
    """Achievable rates of this GPU from the peak microbenchmarks
    (indexer_topk_long_amd/peak/peak.hip): fp8 and bf16 32x32 MFMA loops at
    two waves per SIMD on every CU, alone and with 8 fp32 FMAs issued behind
    each MFMA (the fused scan's head-sum density), and a streaming HBM read.
    Each figure is the best of three timed launches (device events)."""
    import ctypes
    from indexer_topk_long_amd.build import peak_lib_path
    lib = ctypes.CDLL(peak_lib_path())
    lib.ltkpeak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.ltkpeak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks = 256 * 4
    seed = torch.arange(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(blocks * 8, dtype=torch.float32, device="cuda")

    def timed(fn):
        best = None
        for i in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = fn()
            e1.record()
            e1.synchronize()
            if rc != 0:
                raise RuntimeError(f"peak microbenchmark failed ({rc})")
            if i > 0:
                best = e0.elapsed_time(e1) if best is None else min(best, e0.elapsed_time(e1))
        return best

    out = {}
    for kind, name, fl in ((0, "fp8", 131072.0), (1, "bf16", 32768.0)):
        for vpm in (0, 8):
            ms = timed(lambda: lib.ltkpeak_mfma(kind, vpm, blocks, mfma_iters, ctypes.c_void_p(seed.data_ptr()),
                                                ctypes.c_void_p(sink.data_ptr()), stream))
            flops = blocks * 8 * mfma_iters * 8 * fl
            out[f"{name}_mfma_tflops" + ("" if vpm == 0 else f"_with_{vpm}_valu")] = round(flops / (ms * 1e-3) / 1e12, 1)
    buf = torch.empty(read_bytes, dtype=torch.uint8, device="cuda")
    ms = timed(lambda: lib.ltkpeak_read(ctypes.c_void_p(buf.data_ptr()), read_bytes, 256 * 8,
                                        ctypes.c_void_p(sink.data_ptr()), stream))
    out["hbm_read_gbps"] = round(read_bytes / (ms * 1e-3) / 1e9, 1)
    del buf
    return out


def _cores() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] + [1]))
    except Exception:
        return os.cpu_count() or 1


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
    ap.add_argument("--retrieval-sweep", default="", metavar="K1,K2,...",
                    help="retrieval workload only: one line over these k, sample from an earlier batch's results")
    ap.add_argument("--sweep-sample", default="random", choices=["random", "earlier"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--peak", action="store_true", help="print the achievable-peak microbenchmarks and exit")
    ap.add_argument("--no-peak", action="store_true", help="skip the achievable-peak microbenchmarks")
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
              "the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import indexer_topk_long_amd as ltk
    from workloads import WORKLOADS, indexer_workload

    if args.peak:
        print(json.dumps(measure_peaks(torch)), flush=True)
        return

    cfg = WORKLOADS[args.workload]
    if args.prefill_chunks >= 0:
        return bench_prefill_chunks(args)
    if cfg["kind"] == "retrieval":
        return bench_retrieval(args)
    if cfg["kind"] == "decode":
        return bench_decode(args)
    if cfg["kind"] == "dsa":
        return bench_dsa(args)
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
    bytes_q = st.bytes_written / T   # candidates, sample scores and the index output
    full_q = 4.0 * L

    # unfused baseline (full fp32 score matrix + radix select), same inputs
    unf = None
    if args.unfused_steps > 0:
        uws = torch.empty(ltk.workspace_bytes(ltk.KIND_UNFUSED, T, H, D, L, k, 0,
                                              {"f32": 0, "bf16": 1, "fp8": 2}[inp["dtype"]]),
                          dtype=torch.uint8, device="cuda")
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
    peaks = None
    if not args.no_peak:
        log("  achievable-peak microbenchmarks ...")
        peaks = measure_peaks(torch)
    mkey = {"fp8": "fp8_mfma_tflops", "bf16": "bf16_mfma_tflops"}.get(inp["dtype"])

    ctx = "1M" if L == 1 << 20 else f"{L // 1024}K"
    line = {
        "metric": f"scored query-key pairs/s at {ctx} context, k={k}",
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
                     "algorithmic_flops_per_launch": flops,
                     # the same kernel against this GPU's measured MFMA rates
                     # (peak microbenchmarks: MFMA alone, and with the 8 fp32
                     # FMAs per MFMA that the head sum needs)
                     "measured_peak": peaks[mkey] if peaks and mkey else None,
                     "frac_of_measured": round(achieved / peaks[mkey], 4) if peaks and mkey else None,
                     "measured_peak_with_head_sum_valu": peaks.get(mkey + "_with_8_valu") if peaks and mkey else None},
        "measured_peaks": peaks,
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
