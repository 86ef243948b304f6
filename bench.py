"""Benchmark of the CSR graph-attention hot path on one MI355X.

Workload (default): 2^20 rows, power-law in-degrees (pdf exponent 2.1, mean 16, cap
10000), E = 2^24, 4 heads x 64, bf16 q/k/v, fp32 scores and output.  One step is
one pass of the whole path over that graph:

    plan   degree binning (gat_plan_build)
    sddmm  scores[e,h] = <q[row(e),h,:], k[col[e],h,:]>   (gat_sddmm, destination = row of the edge)
    fused  softmax over each row's scores + aggregation of v, hub segments merged
           (gat_fused_layer with scores)

``value`` is edge-heads per second of the whole step (E*H / step time), inputs
resident in HBM before the timed region.  ``roofline`` covers the fused
softmax+aggregate (the dominant and metric kernel): algorithmic bytes per call /
its mean duration measured with HIP events on the launch stream.  ``traffic`` is
the HBM byte count of the same call from rocprofv3 FETCH_SIZE + WRITE_SIZE
(profiles/), scaled by a plain-copy calibration, or null when the kernel sources
changed since the counters were taken.  ``cpu_baseline`` times the CPU oracle on a
bounded prefix of the same graph (every host thread, and one thread).  ``extra`` holds the
other rows of the path timed alone, the unique-bytes lower bound of the fused call and a
streaming device copy measured on the same GPU.

The COO workload c2 (1024 x 128 / 768 x 128 fp32 tables, 16384 edges) has no CSR: its step is
the SDDMM alone and its roofline is the SDDMM's.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4|c5|c3|c2|c1] [--batch B]
                       [--backward]
       python bench.py --workload relation|projection   # the dense l2_p4 block / the projections
       python bench.py --mode copy      # plain-copy calibration target for the counters
       python bench.py --mode gather    # gather calibration target (every table row read once)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
METRIC = "edge-heads/sec for fused CSR edge-softmax+aggregate; % of HBM roofline"
KERNEL_SOURCES = ["common.hpp", "kernels.hpp", "spmm.hpp", "spmm_softagg.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_softagg_c4_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_graph_attention_degree_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per fused call recorded by the counter runs, if they match the current sources."""
    if workload != "c4" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def fused_alg_bytes(n_rows, n_edges, heads, head_dim, feat_bytes):
    """Compulsory bytes of one fused softmax+aggregate call when every gathered source row
    comes from HBM: row_ptr, col_idx, scores, one feature row per edge, the fp32 output."""
    return (4 * (n_rows + 1) + 4 * n_edges + 4 * n_edges * heads + n_edges * heads * head_dim * feat_bytes
            + 4 * n_rows * heads * head_dim)


def copy_calibration(nbytes=1 << 30, reps=3):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read_per_call": nbytes, "bytes_written_per_call": nbytes,
                      "calls": reps}))


def gather_calibration(n=1 << 20, heads=4, head_dim=64, reps=3):
    """Counter calibration target with a known gather footprint: the aggregation kernel on a
    graph of n rows with one edge each, whose columns are a permutation of the n sources, so
    every row of the bf16 [n, heads, head_dim] table (512 MB at the defaults, twice the Infinity
    Cache) is gathered exactly once.  Prints the bytes every call must read and write."""
    import torch
    from sparse_graph_attention_degree_amd import gat
    dev = torch.device("cuda:0")
    r = np.random.default_rng(5)
    rp = torch.arange(n + 1, dtype=torch.int32, device=dev)
    col = torch.from_numpy(r.permutation(n).astype(np.int32)).to(dev)
    wts = torch.ones((n, heads), dtype=torch.float32, device=dev)
    x = torch.randn((n, heads, head_dim), dtype=torch.float32, device=dev).to(torch.bfloat16)
    out = torch.empty((n, heads, head_dim), dtype=torch.float32, device=dev)
    for _ in range(reps):
        gat.gat_aggregate(rp, col, wts, x, out=out)
    torch.cuda.synchronize()
    rows = n * heads * head_dim * 2
    print(json.dumps({"mode": "gather", "kernel": "spmm_short_kernel (aggregate, no plan)", "calls": reps,
                      "gathered_row_bytes_per_call": rows,
                      "bytes_read_per_call": 4 * (n + 1) + 4 * n + 4 * n * heads + rows,
                      "bytes_written_per_call": 4 * n * heads * head_dim}))


def cpu_baseline(g, w, q, k, v, budget_s=12.0, one_thread_s=4.0):
    """The oracle's full layer on a prefix of the graph, grown until it takes ~budget_s on every
    host thread; then a smaller prefix on one thread (~one_thread_s)."""
    import oracle
    from sparse_graph_attention_degree_amd import graphs as G
    orc = oracle.get()

    def run_prefix(target_edges, budget):
        while True:
            rows = int(np.searchsorted(g.row_ptr, target_edges))
            rows = max(1, min(rows, g.n_rows))
            sub_rp, sub_col, _ = G.take_rows(g, np.arange(rows))
            t0 = time.perf_counter()
            orc.layer(sub_rp, sub_col, q[:rows], k, v)
            dt = time.perf_counter() - t0
            e = int(sub_rp[-1])
            if dt >= budget / 4 or rows == g.n_rows:
                return rows, e, dt
            target_edges = int(target_edges * min(16.0, max(2.0, budget / max(dt, 1e-3))))

    threads = orc.num_threads()
    rows, e, dt = run_prefix(1 << 15, budget_s)
    orc.set_num_threads(1)
    try:
        rows1, e1, dt1 = run_prefix(1 << 12, one_thread_s)
    finally:
        orc.set_num_threads(threads)
    return {"value": e * w.heads / dt, "unit": "edge-heads/s", "cores": threads, "kind": "oracle", "host": host_cpu(),
            "sample": f"full layer (sddmm + softmax + aggregate, fp64) on the first {rows} rows "
                      f"({e} edges) of the same graph, {dt:.2f} s",
            "one_thread": {"value": e1 * w.heads / dt1, "unit": "edge-heads/s", "cores": 1,
                           "sample": f"the first {rows1} rows ({e1} edges), {dt1:.2f} s"}}


def host_cpu():
    """Host CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def copy_rate(nbytes=1 << 30, reps=5):
    """Streaming device copy (torch copy_, read + write bytes per second) on this GPU."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / reps
    del src, dst
    return 2 * nbytes / t / 1e9


def bench_backward(gat, rp, col, qd, kd, vd, scores, N, E, H, D, feat_bytes, stream, reps=5):
    """The backward rows over the same graph, each timed alone with HIP events (mean of reps):
    the transposed-graph build, and the full-layer backward (dq, dk, dv)."""
    import torch
    out = {}

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    csc_ws = torch.empty(gat.gat_csc_workspace_bytes(N, N, E, H, D), dtype=torch.uint8, device=vd.device)
    csc = gat.gat_csc_build(rp, col, N, H, D, ws=csc_ws)
    t = timed(lambda: gat.gat_csc_build(rp, col, N, H, D, ws=csc_ws))
    out["csc_build_ms"] = t * 1e3
    plan = gat.gat_plan_build(rp, E, H, D)
    go = torch.randn((N, H, D), dtype=torch.float32, device=vd.device)
    ws = torch.empty(gat.gat_layer_backward_workspace_bytes(E, H), dtype=torch.uint8, device=vd.device)
    t = timed(lambda: gat.gat_fused_layer_backward(rp, col, vd, go, plan, csc, q=qd, k=kd, ws=ws))
    # compulsory bytes: rows gathered per edge -- k (score recompute), v (dL/dalpha), k (dq), q (dk) and
    # grad_out (dv) --, q and grad_out read once per row, dq/dk/dv written, 14 passes over [E,H] fp32
    # arrays (scores, alpha, dL/dalpha, g_s and their CSC copies) and 9 over int32 [E] index arrays
    fb, hd = feat_bytes, H * D
    alg = (4 * E * hd * fb + E * hd * 4 + N * hd * fb + N * hd * 4 + 3 * N * hd * 4 + 14 * 4 * E * H
           + 9 * 4 * E)
    out["layer_backward_ms"] = t * 1e3
    out["layer_backward_edge_heads_per_s"] = E * H / t
    out["layer_backward_alg_bytes"] = alg
    out["layer_backward_gbs"] = alg / t / 1e9
    return out


def bench_relation(args, gat, G):
    """The l2_p4 dense block: one call over `--batch` elements (default: the page's 4) of 24 nodes x
    96 features, 4 heads, 16 pair features."""
    import torch
    sh = dict(G.RELATION_BLOCK)
    if args.batch > 1:
        sh["B"] = args.batch
    B, N, D, H, P = sh["B"], sh["N"], sh["D"], sh["H"], sh["P"]
    nodes, pair, mask, prm = G.make_relation_block(B, N, D, H, P, args.seed, mask="ones")
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    nd, pd, md = t(nodes), t(pair), t(mask)
    pr = {k: t(v) for k, v in prm.items()}
    out = torch.empty_like(nd)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        gat.gat_relation_block(nd, pd, md, pr, out=out)
    # the calls back to back between one pair of events (an event pair around every call adds its
    # own gap to each call)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(args.steps):
        gat.gat_relation_block(nd, pd, md, pr, out=out)
    b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tk = a.elapsed_time(b) * 1e-3 / args.steps
    # arithmetic per element: four D x D projections, pair MLP, q.k and a.v
    flops = B * (4 * 2 * N * D * D + N * N * 2 * (P * P + P * H) + 2 * 2 * H * N * N * (D // H))
    nbytes = B * 4 * (2 * N * D + N * N * P + N * N) + 4 * (4 * D * D + P * P + P + H * P + H + 2 * D)
    cpu = None
    if not args.no_cpu:
        import oracle
        orc = oracle.get()
        k = max(1, min(B, 4))
        t1, reps = time.perf_counter(), 0
        while time.perf_counter() - t1 < 3.0:
            orc.relation_attention(nodes[:k], pair[:k], mask[:k], prm)
            reps += 1
        dt = (time.perf_counter() - t1) / reps
        cpu = {"value": k / dt, "unit": "block elements/s", "cores": 1, "kind": "oracle", "host": host_cpu(),
               "sample": f"{k} elements, {reps} repetitions (the oracle's block is single-threaded)"}
    print(json.dumps({
        "metric": "dense relation-biased attention block (l2_p4): batch elements per second", "value": B / tk,
        "unit": "block elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"relation block: {B} x {N} nodes, {D} features, {H} heads, {P} pair features",
                   "batch": B, "seed": args.seed},
        "roofline": {"bound": "mfma", "achieved": flops / tk / 1e12, "peak": 157.3, "unit": "TFLOP/s",
                     "frac": flops / tk / 1e12 / 157.3, "traffic": None,
                     "kernel": "relation_block_mfma_kernel (one workgroup per element; projections and pair "
                               "MLP on fp32 MFMA 16x16x4, attention on the vector units)"},
        "cpu_baseline": cpu,
        "extra": {"t_call_us": tk * 1e6, "flops_per_call": flops, "hbm_bytes_per_call": nbytes,
                  "hbm_gbs": nbytes / tk / 1e9},
    }))


def bench_projection(args, gat, G):
    """The node projections around the power-law layer (2^20 rows, model dimension 4 x 64 = 256).
    One step = q/k/v projection (bf16 node rows -> three bf16 [rows, 4, 64] arrays, one call),
    the graph attention layer on them, and the output projection of the layer's fp32 output
    (+ bias, fp32).  The layer runs as SDDMM (scores to memory) + fused softmax/aggregation, the
    faster form on this graph: the fully fused q.k layer takes ~9 % longer here (its k and v
    gathers run at 6.3 TB/s against 6.8-7.1 for the two kernels apart) and is timed beside it.
    The degree-binning plan and the row of every edge are built outside the step."""
    import torch
    p = G.PROJECTION
    M, K, H, D = p["M"], p["K"], p["heads"], p["head_dim"]
    w = G.WORKLOADS["c4"]
    g = G.make_graph(w, args.seed)
    x, wqkv, _ = G.make_linear(M, K, 3 * K, seed=args.seed, x_dtype="bf16", bias=False)
    _, wo, bo = G.make_linear(1, K, K, seed=args.seed + 1)
    dev = torch.device("cuda:0")

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    xd, wqkvd, wod, bod = t(x), t(wqkv), t(wo), t(bo)
    rp, col, dst = t(g.row_ptr), t(g.col_idx), t(G.row_of_edge(g.row_ptr))
    E = g.n_edges
    qkv = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    scores = torch.empty((E, H), dtype=torch.float32, device=dev)
    o = torch.empty((M, H, D), dtype=torch.float32, device=dev)
    y = [torch.empty((M, K), dtype=torch.float32, device=dev)]
    plan = gat.gat_plan_build(rp, E, H, D)
    scale = 1.0 / np.sqrt(D)
    stream = torch.cuda.current_stream()

    def qkv_proj():
        gat.gat_linear(xd, wqkvd, n_out=3, y_dtype=torch.bfloat16, out=qkv)

    def layer():
        gat.gat_sddmm(col, dst, qkv[1].view(M, H, D), qkv[0].view(M, H, D), scale=scale, out=scores)
        gat.gat_fused_layer(rp, col, qkv[2].view(M, H, D), scores=scores, out=o, plan=plan)

    def layer_fused_qk():
        gat.gat_fused_layer(rp, col, qkv[2].view(M, H, D), q=qkv[0].view(M, H, D), k=qkv[1].view(M, H, D),
                            scale=scale, out=o, plan=plan)

    def out_proj():
        gat.gat_linear(o.view(M, K), wod, bod, out=y)

    def step():
        qkv_proj()
        layer()
        out_proj()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3

    reps = max(args.steps, 5)
    t_qkv, t_layer, t_out = timed(qkv_proj, reps), timed(layer, reps), timed(out_proj, reps)
    t_layer_qk = timed(layer_fused_qk, reps)
    bytes_qkv = M * K * 2 + 3 * K * K * 2 + 3 * M * K * 2            # x, w, q/k/v (bf16)
    bytes_out = M * K * 4 + K * K * 2 + K * 4 + M * K * 4             # o (fp32), w, bias, y (fp32)
    flops_qkv, flops_out = 2 * M * 3 * K * K, 2 * M * K * K
    cpu = None
    if not args.no_cpu:
        import oracle
        orc = oracle.get()
        rows, reps_c = 4096, 0
        xs = x[:rows]
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < 5.0:
            orc.linear(xs, wqkv)
            orc.linear(xs, wo, bo.astype(np.float64))
            reps_c += 1
        dt = (time.perf_counter() - t1) / reps_c
        cpu = {"value": rows / dt, "unit": "rows/s (both projections)", "cores": orc.num_threads(),
               "kind": "oracle", "host": host_cpu(),
               "sample": f"the q/k/v and output projections of the first {rows} rows, {reps_c} repetitions "
                         f"(the layer between them is the oracle's layer, measured by the default workload)"}
    print(json.dumps({
        "metric": "projected graph attention layer (q/k/v projection, layer, output projection): node rows/s",
        "value": M / (elapsed / args.steps), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"projections around the c4 layer: {M} rows, {K} -> 3 x {K} (bf16) and "
                               f"{K} -> {K} (fp32), {H} heads x {D}, {E} edges", "rows": M, "in_dim": K,
                   "heads": H, "head_dim": D, "n_edges": E, "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": bytes_qkv / t_qkv / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": bytes_qkv / t_qkv / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "linear_wstat_kernel, q/k/v projection (bf16 MFMA 32x32x16, fp32 sums)"},
        "cpu_baseline": cpu,
        "extra": {"t_qkv_us": t_qkv * 1e6, "t_layer_us": t_layer * 1e6, "t_out_us": t_out * 1e6,
                  "layer": "sddmm + fused softmax/aggregate", "t_layer_fused_qk_us": t_layer_qk * 1e6,
                  "qkv_bytes": bytes_qkv, "out_bytes": bytes_out,
                  "qkv_mfma_tflops": flops_qkv / t_qkv / 1e12, "qkv_mfma_frac": flops_qkv / t_qkv / 1e12 / 2500.0,
                  "out_gbs": bytes_out / t_out / 1e9, "out_frac": bytes_out / t_out / 1e9 / HBM_PEAK_GBS,
                  "out_mfma_tflops": flops_out / t_out / 1e12},
    }))


def bench_coo(args, w, gat, G):
    """COO workload: one step = one SDDMM over the edge list."""
    import torch
    si, di, sf, df = G.make_coo(w, args.seed)
    dev = torch.device("cuda:0")
    def t(a):   # uint16 arrays are bfloat16 bit patterns
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    sid, did, sfd, dfd = t(si), t(di), t(sf), t(df)
    E, H, D = w.n_edges, w.heads, w.head_dim
    out = torch.empty((E, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        gat.gat_sddmm(sid, did, sfd, dfd, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        gat.gat_sddmm(sid, did, sfd, dfd, out=out)
        b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_k = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    # launch-bound size: 1000 back-to-back calls timed as one interval
    a0, b0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(1000):
        gat.gat_sddmm(sid, did, sfd, dfd, out=out)
    b0.record(stream)
    torch.cuda.synchronize()
    t_b2b_us = a0.elapsed_time(b0)
    fb = 2 if w.dtype == "bf16" else 4
    alg = 8 * E + 2 * E * H * D * fb + 4 * E * H
    extra = {"t_sddmm_ms": t_k * 1e3, "sddmm_alg_bytes": alg, "sddmm_back_to_back_us": t_b2b_us}
    grad = None
    if args.backward:
        grad = torch.from_numpy(np.random.default_rng(args.seed + 1).standard_normal((E, H)).astype(np.float32)).to(dev)
        ws = torch.empty(gat.gat_sddmm_backward_workspace_bytes(E, w.n_src, w.n_dst, H, D), dtype=torch.uint8,
                         device=dev)
        d_src = torch.empty((w.n_src, H, D), dtype=torch.float32, device=dev)
        d_dst = torch.empty((w.n_dst, H, D), dtype=torch.float32, device=dev)
        bwd = lambda: gat.gat_sddmm_backward(sid, did, sfd, dfd, grad, ws=ws, d_src=d_src, d_dst=d_dst)  # noqa: E731
        for _ in range(max(1, args.warmup)):
            bwd()
        evb = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evb:
            a.record(stream)
            bwd()
            b.record(stream)
        torch.cuda.synchronize()
        t_bwd = float(np.mean([a.elapsed_time(b) for a, b in evb])) * 1e-3
        # per edge: both indices, the gradient and one gathered row of each table; per row: one output row
        bwd_alg = 8 * E + 4 * E * H + 2 * E * H * D * fb + (w.n_src + w.n_dst) * H * D * 4
        bwd_unique = 8 * E + 4 * E * H + (w.n_src + w.n_dst) * H * D * (fb + 4)
        extra.update({"t_sddmm_backward_ms": t_bwd * 1e3, "sddmm_backward_alg_bytes": bwd_alg,
                      "sddmm_backward_gbs": bwd_alg / t_bwd / 1e9,
                      "sddmm_backward_unique_bytes": bwd_unique,
                      "sddmm_backward_unique_gbs": bwd_unique / t_bwd / 1e9,
                      "sddmm_backward_edge_heads_per_s": E * H / t_bwd})
    cpu = None
    if not args.no_cpu:
        import oracle
        orc = oracle.get()
        reps, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < 3.0:
            orc.sddmm(si, di, sf, df)
            reps += 1
        dt = (time.perf_counter() - t1) / reps
        cpu = {"value": E * H / dt, "unit": "edge-heads/s", "cores": orc.num_threads(), "kind": "oracle",
               "host": host_cpu(),
               "sample": f"the whole edge list ({E} edges), {reps} repetitions"}
        if grad is not None:
            gh = grad.cpu().numpy()
            reps, t1 = 0, time.perf_counter()
            while time.perf_counter() - t1 < 3.0:
                orc.sddmm_backward(si, di, sf, df, gh)
                reps += 1
            extra["cpu_sddmm_backward_edge_heads_per_s"] = E * H / ((time.perf_counter() - t1) / reps)
            extra["cpu_sddmm_backward_sample"] = f"the whole edge list, both gradients, {reps} repetitions"
    print(json.dumps({
        "metric": METRIC, "value": E * H / (elapsed / args.steps), "unit": "edge-heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.description, "n_edges": E, "n_src": w.n_src, "n_dst": w.n_dst, "heads": H,
                   "head_dim": D, "features": w.dtype, "seed": args.seed, "step": "sddmm over the edge list"},
        "roofline": {"bound": "hbm", "achieved": alg / t_k / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": alg / t_k / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "sddmm (launch-bound size)" if E < (1 << 20) else "sddmm"},
        "cpu_baseline": cpu,
        "extra": extra,
    }))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4", choices=["c1", "c2", "coo24", "c3", "c4", "c5", "relation",
                                                                "projection"])
    ap.add_argument("--mode", default="bench", choices=["bench", "copy", "gather"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the side measurements")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--batch", type=int, default=1, help="graphs of the workload (seeds seed..seed+B-1) "
                                                          "batched as one block-diagonal graph")
    ap.add_argument("--backward", action="store_true", help="also time the backward: the transposed-graph "
                    "build and the full-layer backward (CSR workloads), the SDDMM backward (COO workloads)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the row range would "
              "shard across GPUs after an all-gather of the feature tables). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.mode == "copy":
        copy_calibration()
        return

    from sparse_graph_attention_degree_amd import gat
    from sparse_graph_attention_degree_amd import graphs as G

    if not os.path.exists(gat.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if args.mode == "gather":
        gather_calibration()
        return

    if args.workload == "relation":
        bench_relation(args, gat, G)
        return
    if args.workload == "projection":
        bench_projection(args, gat, G)
        return
    w = G.WORKLOADS[args.workload]
    if w.kind == "coo":
        bench_coo(args, w, gat, G)
        return
    t0 = time.perf_counter()
    B = max(1, args.batch)
    graphs = [G.make_graph(w, args.seed + b) for b in range(B)]
    q = np.concatenate([G.make_features(w, gb.n_rows, args.seed + b, "q") for b, gb in enumerate(graphs)])
    k = np.concatenate([G.make_features(w, gb.n_src, args.seed + b, "k") for b, gb in enumerate(graphs)])
    v = np.concatenate([G.make_features(w, gb.n_src, args.seed + b, "v") for b, gb in enumerate(graphs)])
    g = graphs[0] if B == 1 else G.block_diagonal(graphs)
    N, E, H, D = g.n_rows, g.n_edges, w.heads, w.head_dim
    feat_bytes = 2 if w.dtype == "bf16" else 4
    log(f"[bench] {args.workload} x {B}: N={N} E={E} H={H} D={D} {w.dtype}; inputs generated in "
        f"{time.perf_counter() - t0:.1f} s")

    dev = torch.device("cuda:0")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    batch_build_ms = None
    if B == 1:
        rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    else:
        # the batch is assembled on the device from the graphs' own arrays (block-diagonal CSR)
        arrays = [to_dev(a) for a in G.batch_arrays(graphs)]
        gat.gat_batch_csr(*arrays)
        a0, b0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a0.record()
        rp, col = gat.gat_batch_csr(*arrays)
        b0.record()
        torch.cuda.synchronize()
        batch_build_ms = a0.elapsed_time(b0)
    dst = to_dev(G.row_of_edge(g.row_ptr))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    scores = torch.empty((E, H), dtype=torch.float32, device=dev)
    out = torch.empty((N, H, D), dtype=torch.float32, device=dev)
    ws = torch.empty(gat.gat_plan_workspace_bytes(N, E, H, D), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    n_ev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_ev)]

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        plan = gat.gat_plan_build(rp, E, H, D, ws=ws)
        if evs:
            evs[1].record(stream)
        gat.gat_sddmm(col, dst, kd, qd, out=scores)
        if evs:
            evs[2].record(stream)
        gat.gat_fused_layer(rp, col, vd, scores=scores, out=out, plan=plan)
        if evs:
            evs[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    t_plan = np.mean([e[0].elapsed_time(e[1]) for e in ev]) * 1e-3
    t_sddmm = np.mean([e[1].elapsed_time(e[2]) for e in ev]) * 1e-3
    t_fused = np.mean([e[2].elapsed_time(e[3]) for e in ev]) * 1e-3
    ms_per_step = elapsed / args.steps * 1e3
    value = E * H / (elapsed / args.steps)

    alg = fused_alg_bytes(N, E, H, D, feat_bytes)
    achieved = alg / t_fused / 1e9
    traffic = read_traffic(args.workload)

    # lower bound: every distinct source row read once (the rest as in the algorithmic count)
    n_distinct = int(np.count_nonzero(np.bincount(g.col_idx, minlength=g.n_src))) if E else 0
    unique = alg - E * H * D * feat_bytes + n_distinct * H * D * feat_bytes
    fused_ms = [e[2].elapsed_time(e[3]) for e in ev]
    extra = {"t_plan_ms": t_plan * 1e3, "t_sddmm_ms": t_sddmm * 1e3, "t_fused_ms": t_fused * 1e3,
             "t_fused_median_ms": float(np.median(fused_ms)), "t_fused_min_ms": float(np.min(fused_ms)),
             "fused_edge_heads_per_s": E * H / t_fused,
             "fused_alg_bytes": alg,
             "fused_unique_bytes": unique,
             "fused_unique_gbs": unique / t_fused / 1e9,
             # the same call priced on unique bytes (every distinct source row read once): a
             # schedule that reused every gathered row from cache would reach this fraction
             "fused_unique_frac": unique / t_fused / 1e9 / HBM_PEAK_GBS,
             # The SDDMM reads two rows per edge, but the destination (query) row repeats along each
             # CSR row and stays in cache, so only the k gathers reach memory: that count is its
             # HBM rate; the two-rows-per-edge count is an effective rate, above the HBM peak here.
             "sddmm_hbm_bytes": 8 * E + E * H * D * feat_bytes + 4 * E * H,
             "sddmm_hbm_gbs": (8 * E + E * H * D * feat_bytes + 4 * E * H) / t_sddmm / 1e9,
             "sddmm_effective_two_row_gbs": (8 * E + 2 * E * H * D * feat_bytes + 4 * E * H) / t_sddmm / 1e9,
             "kernel_source_sha256": kernel_source_digest()}
    if batch_build_ms is not None:
        extra["batch_graphs"] = B
        extra["batch_build_ms"] = batch_build_ms
    if E * H < (1 << 22):
        # launch-bound sizes: the whole step captured once in a HIP graph, 100 replays timed as one
        graph = torch.cuda.CUDAGraph()
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        graph.replay()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(100):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        extra["step_graph_replay_us"] = a.elapsed_time(b) * 10.0   # ms for 100 replays -> us per replay
        extra["step_graph_replay_edge_heads_per_s"] = E * H / (a.elapsed_time(b) * 1e-5)
        # launch-bound sizes: 1000 back-to-back planned fused calls timed as one interval
        plan = gat.gat_plan_build(rp, E, H, D, ws=ws)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(1000):
            gat.gat_fused_layer(rp, col, vd, scores=scores, out=out, plan=plan)
        b.record(stream)
        torch.cuda.synchronize()
        extra["fused_back_to_back_us"] = a.elapsed_time(b)  # ms for 1000 calls = us per call
    if not args.no_extra:
        cp = copy_rate()
        extra["copy_gbs"] = cp
        extra["fused_frac_of_copy"] = achieved / cp

    if not args.no_extra:
        # the other rows of the path, each timed alone over the same graph (5 calls, HIP events)
        plan = gat.gat_plan_build(rp, E, H, D, ws=ws)
        alpha = torch.empty_like(scores)
        gat.gat_edge_softmax(rp, scores, out=alpha, plan=plan)
        row_bytes = {
            "edge_softmax": (4 * (N + 1) + 8 * E * H,
                             lambda: gat.gat_edge_softmax(rp, scores, out=alpha, plan=plan)),
            "aggregate": (fused_alg_bytes(N, E, H, D, feat_bytes),
                          lambda: gat.gat_aggregate(rp, col, alpha, vd, out=out, plan=plan)),
            "full_layer_qk_on_the_fly": (4 * (N + 1) + 4 * E + N * H * D * feat_bytes
                                         + 2 * E * H * D * feat_bytes + 4 * N * H * D,
                                         lambda: gat.gat_fused_layer(rp, col, vd, q=qd, k=kd, out=out, plan=plan)),
            "fused_no_plan": (alg, lambda: gat.gat_fused_layer(rp, col, vd, scores=scores, out=out)),
        }
        for name, (nbytes, fn) in row_bytes.items():
            fn()
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s0.record(stream)
            reps = 5
            for _ in range(reps):
                fn()
            s1.record(stream)
            torch.cuda.synchronize()
            t = s0.elapsed_time(s1) * 1e-3 / reps
            extra[f"{name}_ms"] = t * 1e3
            extra[f"{name}_edge_heads_per_s"] = E * H / t
            extra[f"{name}_alg_bytes"] = nbytes
            extra[f"{name}_gbs"] = nbytes / t / 1e9

    if args.backward:
        extra.update(bench_backward(gat, rp, col, qd, kd, vd, scores, N, E, H, D, feat_bytes, stream))

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a prefix sample ...")
        cpu = cpu_baseline(g, w, q, k, v)

    rec = {
        "metric": METRIC, "value": value, "unit": "edge-heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.description if B == 1 else f"{B} graphs of: {w.description}", "n_rows": N,
                   "n_edges": E, "heads": H, "head_dim": D, "features": w.dtype, "accumulate": "f32",
                   "seed": args.seed, "batch": B,
                   "step": "plan (degree binning) + sddmm q.k + fused softmax/aggregate of v"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "fused softmax+aggregate (gat_fused_layer with scores: segment, short-row and "
                               "hub-merge kernels)",
                     "bytes": "algorithmic: row_ptr, col_idx, scores, one gathered source row per edge, the "
                              "fp32 output; these are bytes past the L2 (the Infinity Cache serves part of "
                              "them), not bytes on the HBM bus; extra.fused_unique_frac prices the same call "
                              "on each distinct row read once"},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
