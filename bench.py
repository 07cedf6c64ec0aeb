#!/usr/bin/env python3
"""Benchmark of the compressed-attention hot path on one MI355X.

Default workload: one CSA decode step at 128K context, batch 32 — indexer
scores (64 heads x 128 dims, bf16) over 32768 compressed entries per sequence,
top-512 selection, then attention of 64 query heads (one KV head, head dim
512) over the 512 selected entries plus a 128-token window with sinks.
Throughput = query tokens per second of the whole step, inputs resident in
HBM. Two independent input sets alternate between steps so the working set is
larger than the 256 MB Infinity Cache.

Other workloads (--workload): hca_decode (HCA at 1M context, batch 16),
pair_1m (CSA with an MXFP4 indexer plus HCA at 1M context, batch 8),
indexer_fp8_prefill (the fp8 indexer of a 4096-token prefill chunk at 64K
context with 64 heads x 128 dims), compress (the compressor's bandwidth) and
csa_decode_state (the CSA decode step with the state cache: token append and
block compression, then indexer top-k and attention with a position per
sequence around 128K) and indexer_bf16_scores (the literal fp8 4 x 32 indexer
and top-1024 of a 4096-token prefill chunk at 64K with f32 and with bf16
scores: speedup and recall), csa_attn_bwd (the attention backward on the
2048-token prefill and on the 4096-token chunk at 64K) and csa_prefill (one
CSA layer on the 4096-token chunk at 64K: compress, index_topk, sparse_attn).

Prints one JSON line. The CPU baseline times the CPU oracle (test
infrastructure) on a bounded sample of the same workload on the host cores.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
# Seconds of back-to-back work before any timed region: after an idle spell
# the GPU's clocks ramp up over the first few tens of milliseconds of load
# (measured: the fp8 prefill indexer 580 -> 400 -> 360 us per launch over its
# first 40 launches, then flat for seconds; the decode step 98.5 -> 94.4 us),
# so a handful of warmup steps would time the ramp, not the kernels.
SETTLE_S = 0.25
SETTLE_NOTE = "after %.2f s of back-to-back work (clock ramp-up)" % SETTLE_S


def settle(torch, fn, seconds=SETTLE_S):
    """Call fn(k) back to back until `seconds` have passed (synchronizing
    every 8 calls); returns the number of calls."""
    t_end = time.perf_counter() + seconds
    k = 0
    while True:
        for _ in range(8):
            fn(k)
            k += 1
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            return k


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="csa_decode",
                    choices=["csa_decode", "hca_decode", "pair_1m", "indexer_fp8_prefill", "compress",
                             "csa_decode_state", "indexer_bf16_scores", "csa_attn_bwd", "csa_prefill"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run the 1 GiB copy (calibration run for HBM byte counters)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target length of the CPU-oracle sample")
    return ap.parse_args()


# --------------------------------------------------------------------------
def fused_cols(topk):
    """Entries per chunk of the fused indexer + chunk top-k (0: k too large)."""
    return 2048 if topk <= 512 else 4096 if topk <= 1024 else 0


def fused(s):
    """Whether csa_index_topk runs fused for shape s (one query per indexer
    workgroup and k at most a quarter of a chunk)."""
    return (s.H_I >= 64 or s.Lq == 1) and fused_cols(s.topk) > 0


def csa_decode_setup(torch, csa, wl, shape, seeds, dev):
    sets = []
    for sd in seeds:
        x = wl.make_inputs(shape, sd, device=dev)
        B, Lq = shape.B, shape.Lq
        x["scores"] = torch.empty((B, Lq, shape.N_cap), dtype=torch.float32, device=dev)
        x["idx"] = torch.empty((B, Lq, shape.topk), dtype=torch.int32, device=dev)
        tb = csa.topk_ws_bytes(B, Lq, shape.q_pos0, shape.m, shape.topk)
        x["topk_ws"] = torch.empty((tb + 15) // 16 * 4, dtype=torch.float32, device=dev)
        if fused(shape):
            cb = csa.index_candidates_bytes(B, Lq, shape.q_pos0, shape.m, shape.topk)
            x["cand"] = torch.empty((cb + 15) // 16 * 4, dtype=torch.float32, device=dev)
        nb = csa.sparse_attn_ws_bytes(B, Lq, shape.H, shape.D, shape.topk, shape.W)
        x["ws"] = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=dev)
        x["out"] = torch.empty_like(x["q"])
        x["lse"] = torch.empty((B, Lq, shape.H), dtype=torch.float32, device=dev)
        sets.append(x)
    return sets


def hca_setup(torch, csa, wl, shape, seeds, dev):
    sets = []
    for sd in seeds:
        x = wl.make_inputs(shape, sd, device=dev)
        nb = csa.hca_attn_ws_bytes(shape.B, shape.Lq, shape.q_pos0, shape.m, shape.H, shape.D, shape.W)
        x["ws"] = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=dev)
        x["out"] = torch.empty_like(x["q"])
        x["lse"] = torch.empty((shape.B, shape.Lq, shape.H), dtype=torch.float32, device=dev)
        sets.append(x)
    return sets


# ---------------------------------------------------------- algorithmic bytes
def idx_row_bytes(s):
    return {"bf16": 2, "fp8": 1, "f32": 4}.get(s.idx, 0) * s.d_I or (s.d_I // 2 + s.d_I // 32)


def index_qk_bytes(s):
    """k_I rows of visible entries + q_I + head weights + scores written once."""
    vis = sum((s.q_pos0 + i + 1) // s.m for i in range(s.Lq))
    n_last = (s.q_pos0 + s.Lq) // s.m
    kb = s.B * n_last * idx_row_bytes(s)
    qb = s.B * s.Lq * s.H_I * idx_row_bytes(s)
    return kb + qb + s.B * s.Lq * s.H_I * 4 + s.B * vis * 4


def index_qk_flops(s):
    vis = sum((s.q_pos0 + i + 1) // s.m for i in range(s.Lq))
    return 2.0 * s.H_I * s.d_I * s.B * vis


def sparse_attn_bytes(s):
    kvb = 2 if s.kv == "bf16" else 4
    rows = s.topk + s.W
    return s.B * s.Lq * (rows * 2 * s.D * kvb + 2 * s.H * s.D * kvb + s.H * 4 + s.topk * 4)


def index_cand_bytes(s):
    """Fused indexer: k_I rows, q_I and head weights read once, and the
    per-chunk candidate lists (8 bytes a slot) written once."""
    n_last = (s.q_pos0 + s.Lq) // s.m
    nchunks = -(-n_last // fused_cols(s.topk))
    kb = s.B * n_last * idx_row_bytes(s)
    qb = s.B * s.Lq * s.H_I * idx_row_bytes(s)
    return kb + qb + s.B * s.Lq * s.H_I * 4 + s.B * s.Lq * nchunks * s.topk * 8


def topk_merge_bytes(s):
    """Merge levels of the fused lists (groups of max(2, 8192 // k) lists per
    workgroup): every level reads its input lists and writes its output
    lists, the last one the indices."""
    n = -(-((s.q_pos0 + s.Lq) // s.m) // fused_cols(s.topk))
    g = max(2, 8192 // s.topk)
    total = 0
    while True:
        nout = -(-n // g)
        total += s.B * s.Lq * n * s.topk * 8 + (s.B * s.Lq * nout * s.topk * 8 if nout > 1 else 0)
        n = nout
        if n <= 1:
            break
    return total + s.B * s.Lq * s.topk * 4


def topk_bytes(s):
    vis = sum((s.q_pos0 + i + 1) // s.m for i in range(s.Lq))
    return s.B * vis * 4 + s.B * s.Lq * s.topk * 4


def hca_bytes(s):
    kvb = 2 if s.kv == "bf16" else 4
    n = (s.q_pos0 + 1) // s.m
    return s.B * s.Lq * ((n + s.W) * 2 * s.D * kvb + 2 * s.H * s.D * kvb + s.H * 4)


# HBM bytes per dispatch of the dominant kernel from rocprofv3 counter runs
# (FETCH_SIZE, then WRITE_SIZE), each scaled by what the counter reads for a
# plain copy of known size; the summary files under profiles/ record the
# values with a SHA-256 of the kernel's sources, and the figure is reported
# only while those sources are unchanged.
TRAFFIC_FILES = {("csa_decode", "index_cand"): "index_qk_fused_csa_decode_128k_b32_traffic.md"}


def kernel_sources_sha(names):
    """SHA-256 over the named csrc/ files, in order."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_attention_16_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    name = TRAFFIC_FILES.get((workload, kernel))
    if not name:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            fields = dict(line.strip()[2:].split(": ", 1) for line in f if line.startswith("- ") and ": " in line)
        srcs = fields["kernel sources"].split(", ")
        if kernel_sources_sha(srcs) != fields["sources sha256"]:
            return None
        return float(fields["traffic bytes per dispatch"])
    except (OSError, KeyError, ValueError):
        return None


# Compressor workloads: (name, T tokens of one sequence, D, m); bf16 K and V.
COMPRESS_CASES = [("ctx64k_d128_m4", 65536, 128, 4), ("seq1m_d512_m4", 1 << 20, 512, 4),
                  ("seq1m_d512_m128", 1 << 20, 512, 128)]


def bench_compress(args, torch, csa, dev):
    """HBM bandwidth of csa_compress: K and V rows read once, compressed rows
    written once (bytes = 2*T*D*2 + 2*(T/m)*D*2), timed with HIP-graph replays
    of back-to-back calls."""
    out = {}
    for name, T, D, m in COMPRESS_CASES:
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        k_raw = torch.randn((1, T, D), generator=gen, device=dev).to(torch.bfloat16)
        v_raw = torch.randn((1, T, D), generator=gen, device=dev).to(torch.bfloat16)
        w_gate = torch.randn((D,), generator=gen, device=dev) / D ** 0.5
        k_c = torch.empty((1, T // m, D), dtype=torch.bfloat16, device=dev)
        v_c = torch.empty_like(k_c)
        for _ in range(max(args.warmup, 2)):
            csa.compress(k_raw, v_raw, w_gate, m, 0, k_c, v_c)
        torch.cuda.synchronize()
        reps = max(args.steps // 5, 2)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                csa.compress(k_raw, v_raw, w_gate, m, 0, k_c, v_c)
        g.replay()
        torch.cuda.synchronize()
        settle(torch, lambda k: g.replay())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = 1000.0 * e0.elapsed_time(e1) / (5 * reps)
        nbytes = 2 * T * D * 2 + 2 * (T // m) * D * 2
        out[name] = {"us": round(us, 2), "gbs": round(nbytes / us / 1e3, 1), "bytes": nbytes}
        del k_raw, v_raw, k_c, v_c
        torch.cuda.empty_cache()
    main_case = out["seq1m_d512_m4"]
    roof = {"bound": "hbm", "achieved": main_case["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(main_case["gbs"] / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "compress",
            "bytes_per_launch": main_case["bytes"]}
    result = {
        "metric": "compressor HBM GB/s (1M tokens, D=512, m=4)", "value": main_case["gbs"], "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(main_case["us"] / 1000.0, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) raw K/V rows)",
        "config": {"workload": "compress_seq1m_d512_m4", "cases": {c[0]: {"tokens": c[1], "head_dim": c[2], "m": c[3]}
                                                                  for c in COMPRESS_CASES}},
        "roofline": roof, "cases": out,
        "timing": "HIP-graph replays of back-to-back calls per case, " + SETTLE_NOTE,
        "copy_ceiling_gbs": copy_ceiling(torch, dev), "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _oracle_compress_baseline(torch, dev, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _oracle_compress_baseline(torch, dev, seconds):
    """The oracle compressor (float64) on the main case's inputs (1M tokens,
    D = 512, m = 4, same seed), 8192 tokens at a time until `seconds` of work;
    GB/s counts the same algorithmic bytes as the GPU figure."""
    import numpy as np
    from oracle import compress as ocmp, formats
    T, D, m = 1 << 20, 512, 4
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    k_raw = torch.randn((1, T, D), generator=gen, device=dev).to(torch.bfloat16)
    v_raw = torch.randn((1, T, D), generator=gen, device=dev).to(torch.bfloat16)
    w_gate = (torch.randn((D,), generator=gen, device=dev) / D ** 0.5).cpu().numpy().astype(np.float64)

    def bf(t_):
        return formats.bf16_to_f64(t_.view(torch.int16).numpy().view(np.uint16))

    done, spent, step = 0, 0.0, 8192
    while done < T and (done == 0 or spent < seconds):
        kr, vr = bf(k_raw[0, done:done + step].cpu()), bf(v_raw[0, done:done + step].cpu())
        t0 = time.perf_counter()
        ocmp.compress(kr, vr, w_gate, m, done)
        spent += time.perf_counter() - t0
        done += step
    nbytes = 2 * done * D * 2 + 2 * (done // m) * D * 2
    del k_raw, v_raw
    torch.cuda.empty_cache()
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": "%d of %d tokens of compress_seq1m_d512_m4, %.1f s of oracle work (numpy float64)"
                      % (done, T, spent)}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(blas) if blas else 1
    except Exception:
        return 1


def _oracle_prefill_indexer_baseline(s, x, seconds):
    """The oracle's fp8 64 x 128 indexer scores, query by query of the
    prefill chunk, until `seconds` of work."""
    import numpy as np
    import torch
    from oracle import formats, indexer as oidx

    def f8(t_):
        return formats.e4m3fn_to_f64(t_.view(torch.uint8).numpy())

    ki = f8(x["k_i"][0].cpu())
    qi, wi = x["q_i"][0].cpu(), x["w_i"][0].cpu()
    done, spent = 0, 0.0
    while done < s.Lq and (done == 0 or spent < seconds):
        n = (s.q_pos0 + done + 1) // s.m
        qd, wd = f8(qi[done]), wi[done].numpy().astype(np.float64)
        t0 = time.perf_counter()
        oidx.index_scores(qd, wd, ki[:n])
        spent += time.perf_counter() - t0
        done += 1
    return {"value": round(done / spent, 4), "unit": "query-tok/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": "%d of %d query rows of %s, %.1f s of oracle work (numpy float64)"
                      % (done, s.Lq, s.name, spent)}


def bench_state_decode(args, torch, csa, wl, dev):
    """The CSA decode step with the state cache at 128K context, batch 32:
    csa_state_append (each token into its sequence's 128-slot ring; the
    sequences whose token completes a block of 4 compress it, a quarter of the
    batch per step), then csa_index_topk_varlen and csa_sparse_attn_varlen
    with one position per sequence (131071 - 37 b: lengths differ, and
    b % 4 == 0 completes a block). HIP-graph replays of the whole step, two
    input sets alternating."""
    s = wl.CFG2
    R, d_i = s.T_raw, s.d_I
    pos_l = [s.q_pos0 - 37 * b for b in range(s.B)]
    q_pos_max = max(pos_l)
    sets = []
    for sd in (wl.SEEDS["2"], 1000 + wl.SEEDS["2"]):
        x = wl.make_inputs(s, sd, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(sd + 5)
        bf = lambda *sh: torch.randn(sh, generator=gen, device=dev).to(torch.bfloat16)
        x.update(pos=torch.tensor(pos_l, dtype=torch.int64, device=dev), k_new=bf(s.B, s.D), v_new=bf(s.B, s.D),
                 ki_new=bf(s.B, d_i), ki_ring=bf(s.B, R, d_i),
                 idx=torch.empty((s.B, 1, s.topk), dtype=torch.int32, device=dev),
                 out=torch.empty_like(x["q"]), lse=torch.empty((s.B, 1, s.H), dtype=torch.float32, device=dev))
        ib = csa.index_topk_ws_bytes(s.B, 1, q_pos_max, s.m, s.N_cap, s.topk)
        x["iws"] = torch.empty((ib + 15) // 16 * 4, dtype=torch.float32, device=dev)
        ab = csa.sparse_attn_ws_bytes(s.B, 1, s.H, s.D, s.topk, s.W)
        x["aws"] = torch.empty((ab + 15) // 16 * 4, dtype=torch.float32, device=dev)
        sets.append(x)
    torch.cuda.synchronize()

    def launch(label, x):
        if label == "state_append":
            csa.state_append(x["pos"], x["k_new"], x["v_new"], x["w_gate"], s.m, x["k_raw"], x["v_raw"], x["k_c"],
                             x["v_c"], x["ki_new"], x["ki_ring"], x["k_i"], None, s.idx)
        elif label == "index_topk":
            csa.index_topk_varlen(x["q_i"], x["w_i"], x["k_i"], s.topk, x["pos"], q_pos_max, s.m, s.idx,
                                  ws=x["iws"], out=x["idx"])
        else:
            csa.sparse_attn_varlen(x["q"], x["k_c"], x["v_c"], x["idx"], x["k_raw"], x["v_raw"], s.W, x["sink"],
                                   x["pos"], q_pos_max, ws=x["aws"], out=x["out"], lse=x["lse"])

    labels = ["state_append", "index_topk", "sparse_attn"]
    for k in range(args.warmup):
        for l in labels:
            launch(l, sets[k % 2])
    torch.cuda.synchronize()
    graphs = []
    for k in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in labels:
                launch(l, sets[k])
        graphs.append(g)
    settle(torch, lambda k: graphs[k % 2].replay())
    breakdown = {}
    for l in labels:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(args.steps):
            launch(l, sets[k % 2])
        e1.record()
        torch.cuda.synchronize()
        breakdown[l] = round(1000.0 * e0.elapsed_time(e1) / args.steps, 2)
    for k in range(args.warmup):
        graphs[k % 2].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        graphs[k % 2].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps

    # algorithmic bytes of the index_topk call: the visible k_I rows of each
    # sequence, q_I and head weights, the candidate lists written and read,
    # the indices written
    vis = [(p + 1) // s.m for p in pos_l]
    nch = -(-max(vis) // fused_cols(s.topk))
    row = idx_row_bytes(s)
    ib = sum(vis) * row + s.B * s.H_I * (row + 4) + 2 * s.B * nch * s.topk * 8 + s.B * s.topk * 4
    roof = {"bound": "hbm", "achieved": ib / (breakdown["index_topk"] * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
            "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof.update(traffic=None, kernel="index_topk (fused indexer + merge)", bytes_per_launch=ib)
    roof = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()}
    result = {
        "metric": "CSA decode query-tok/s with state cache @128K ctx", "value": round(s.B / (ms / 1000.0), 1),
        "unit": "query-tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) caches, tokens and queries, random-init indexer; no weights or datasets)",
        "config": {"workload": "csa_decode_state_128k_b32_bf16", "batch": s.B,
                   "positions": "131071 - 37 b", "ring_slots": R, "m": s.m, "compressing_per_step": sum(
                       1 for p in pos_l if (p + 1) % s.m == 0), "heads": s.H, "head_dim": s.D,
                   "indexer": "%dx%d %s" % (s.H_I, s.d_I, s.idx), "topk": s.topk, "window": s.W},
        "roofline": roof, "breakdown_us": breakdown,
        "timing": "value/ms_per_step: HIP-graph replays of the whole step; breakdown_us: back-to-back calls "
                  "between HIP events; " + SETTLE_NOTE,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline("csa_decode_state_128k_b32_bf16", [(s, sets[0])], args.cpu_seconds,
                                              query_fn=lambda s_, x_, b_: _oracle_state_query(s_, x_, b_, pos_l[b_]))
    print(json.dumps(result), flush=True)


def bench_bf16_scores(args, torch, csa, wl, dev):
    """csa_index_topk_ex on the prefill chunk (4096 queries at 61440.., 16384
    compressed entries, literal fp8 indexer 4 x 32, top-1024, N(0,1) inputs)
    with f32 and with bf16 scores: the scores make a round trip through HBM
    (268 MB of f32 written and read), so their precision sets the time.
    Recall = mean over queries of |bf16 selection & f32 selection| / k.
    HIP-graph replays of back-to-back calls, two input sets alternating."""
    from dataclasses import replace
    s = replace(wl.CFG3, exact=False)
    xs = []
    for sd in (wl.SEEDS["3"], 1000 + wl.SEEDS["3"]):
        gen = torch.Generator(device=dev)
        gen.manual_seed(sd)
        x = wl.indexer_inputs(s, gen, dev)
        nb = csa.index_topk_ws_bytes(s.B, s.Lq, s.q_pos0, s.m, s.N_cap, s.topk)
        x["ws"] = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=dev)
        x["out"] = {p: torch.empty((s.B, s.Lq, s.topk), dtype=torch.int32, device=dev) for p in ("f32", "bf16")}
        xs.append(x)

    for x in xs:
        x["sc"] = {"f32": torch.empty((s.B, s.Lq, s.N_cap), dtype=torch.float32, device=dev),
                   "bf16": torch.empty((s.B, s.Lq, (s.N_cap + 1) // 2 * 2), dtype=torch.bfloat16, device=dev)}

    def call(x, prec):
        csa.index_topk_ex(x["q_i"], x["w_i"], x["k_i"], s.topk, s.q_pos0, s.m, s.idx, prec, None, x["q_i_scale"],
                          x["k_i_scale"], ws=x["ws"], out=x["out"][prec])

    def scores_only(x, prec):
        csa.index_scores_ex(x["q_i"], x["w_i"], x["k_i"], s.q_pos0, s.m, s.idx, prec, None, x["q_i_scale"],
                            x["k_i_scale"], out=x["sc"][prec])

    us, us_idx = {}, {}
    for prec in ("f32", "bf16"):
        for k in range(4):
            scores_only(xs[k % 2], prec)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(10):
                scores_only(xs[k % 2], prec)
        g.replay()
        torch.cuda.synchronize()
        settle(torch, lambda k: g.replay())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us_idx[prec] = 1000.0 * e0.elapsed_time(e1) / 50
    for prec in ("f32", "bf16"):
        for k in range(max(args.warmup, 2)):
            call(xs[k % 2], prec)
        torch.cuda.synchronize()
        reps = 10
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(reps):
                call(xs[k % 2], prec)
        g.replay()
        torch.cuda.synchronize()
        settle(torch, lambda k: g.replay())
        n_rep = max(1, args.steps // reps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_rep):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us[prec] = 1000.0 * e0.elapsed_time(e1) / (n_rep * reps)
    # recall of the bf16 selection against the f32 one (last call of each on set 1)
    a, b = xs[1]["out"]["f32"][0], xs[1]["out"]["bf16"][0]
    mark = torch.zeros((s.Lq, s.N_cap + 1), dtype=torch.int8, device=dev)
    mark.scatter_(1, torch.where(a >= 0, a, s.N_cap).long(), 1)
    hit = torch.gather(mark, 1, torch.where(b >= 0, b, s.N_cap).long()).float()
    valid = (a >= 0).float().sum(1).clamp(min=1)
    recall = float(((hit * (b >= 0).float()).sum(1) / valid).mean())

    vis = sum((s.q_pos0 + i + 1) // s.m for i in range(s.Lq))
    n_last = (s.q_pos0 + s.Lq) // s.m
    base = s.B * n_last * s.d_I + s.B * s.Lq * s.H_I * (s.d_I + 4) + s.B * s.Lq * s.topk * 4
    nbytes = {p: base + 2 * s.B * vis * (4 if p == "f32" else 2) for p in ("f32", "bf16")}
    roof = {"bound": "hbm", "achieved": nbytes["bf16"] / (us["bf16"] * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
            "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof.update(traffic=None, kernel="index_topk_ex bf16 (indexer scores + chunk top-k + merge)",
                bytes_per_launch=nbytes["bf16"])
    roof = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()}
    result = {
        "metric": "indexer top-k query-tok/s with bf16 scores (prefill chunk 4096 @64K)",
        "value": round(s.Lq / (us["bf16"] * 1e-6), 1), "unit": "query-tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us["bf16"] / 1000.0, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic (seeded N(0,1) indexer queries and keys in e4m3fn, random head weights)",
        "config": {"workload": "indexer_bf16_scores_chunk4096_ctx64k_fp8", "query_chunk": s.Lq,
                   "context": s.q_pos0 + s.Lq, "compressed_entries": s.N_cap,
                   "indexer": "%dx%d %s" % (s.H_I, s.d_I, s.idx), "topk": s.topk},
        "roofline": roof,
        "us_per_call": {p: round(v, 2) for p, v in us.items()},
        "speedup_bf16_over_f32": round(us["f32"] / us["bf16"], 3), "recall_vs_f32": round(recall, 5),
        "indexer_scores_us": {p: round(v, 2) for p, v in us_idx.items()},
        "indexer_speedup_bf16_over_f32": round(us_idx["f32"] / us_idx["bf16"], 3),
        "indexer_scores_gbs": {p: round((base - s.B * s.Lq * s.topk * 4 + s.B * vis * (4 if p == "f32" else 2))
                                        / (v * 1e-6) / 1e9, 1) for p, v in us_idx.items()},
        "timing": "HIP-graph replays of back-to-back calls, two input sets alternating, " + SETTLE_NOTE,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _oracle_bf16_baseline(s, xs[0], args.cpu_seconds)
    print(json.dumps(result), flush=True)


def bench_prefill(args, torch, csa, wl, dev):
    """One CSA layer on a 4096-token prefill chunk at positions 61440..65535
    of a 64K context (config-3 shapes: bf16 KV, H = 4, D = 128, 16384
    compressed entries, literal fp8 indexer 4 x 32, top-1024, W = 128, N(0,1)
    inputs): csa_compress folds the chunk's own 4096 tokens (K, V and the
    indexer keys, stored as e4m3fn) into entries 15360..16383, csa_index_topk
    scores those and the earlier entries and selects, csa_sparse_attn attends. Step time:
    HIP-graph replays of the three calls, two input sets alternating; per-call
    times: back-to-back launches between HIP events."""
    from dataclasses import replace
    s = replace(wl.CFG3, exact=False)
    chunk = slice(s.comp_pos0 - s.raw_pos0, s.comp_pos0 - s.raw_pos0 + s.T_comp)
    xs = []
    for sd in (wl.SEEDS["3"], 1000 + wl.SEEDS["3"]):
        x = wl.make_inputs(s, sd, device=dev)
        x["kraw_chunk"] = x["k_raw"][:, chunk].contiguous()
        x["vraw_chunk"] = x["v_raw"][:, chunk].contiguous()
        x["kiraw_chunk"] = wl.chunk_index_keys(s, sd, dev)
        nb = csa.index_topk_ws_bytes(s.B, s.Lq, s.q_pos0, s.m, s.N_cap, s.topk)
        x["tws"] = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=dev)
        x["idx"] = torch.empty((s.B, s.Lq, s.topk), dtype=torch.int32, device=dev)
        nb = csa.sparse_attn_ws_bytes(s.B, s.Lq, s.H, s.D, s.topk, s.W)
        x["aws"] = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=dev)
        x["out"] = torch.empty_like(x["q"])
        x["lse"] = torch.empty((s.B, s.Lq, s.H), dtype=torch.float32, device=dev)
        xs.append(x)
    torch.cuda.synchronize()

    calls = {
        "compress": lambda x: csa.compress(x["kraw_chunk"], x["vraw_chunk"], x["w_gate"], s.m, s.comp_pos0,
                                           x["k_c"], x["v_c"], ki_raw=x["kiraw_chunk"], ki_c=x["k_i"],
                                           ki_scale=x["k_i_scale"], idx_fmt=s.idx),
        "index_topk": lambda x: csa.index_topk(x["q_i"], x["w_i"], x["k_i"], s.topk, s.q_pos0, s.m, s.idx,
                                               x["q_i_scale"], x["k_i_scale"], ws=x["tws"], out=x["idx"]),
        "sparse_attn": lambda x: csa.sparse_attn(x["q"], x["k_c"], x["v_c"], x["idx"], x["k_raw"], x["v_raw"],
                                                 s.raw_pos0, s.W, x["sink"], s.q_pos0, ws=x["aws"], out=x["out"],
                                                 lse=x["lse"]),
    }

    def step(k):
        for f in calls.values():
            f(xs[k % 2])

    for k in range(max(args.warmup, 2)):
        step(k)
    torch.cuda.synchronize()
    graphs = []
    for k in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(k)
        graphs.append(g)
    settle(torch, lambda k: graphs[k % 2].replay())
    reps = max(4, min(args.steps, 20))
    breakdown = {}
    for name, f in calls.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(reps):
            f(xs[k % 2])
        e1.record()
        torch.cuda.synchronize()
        breakdown[name] = round(1000.0 * e0.elapsed_time(e1) / reps, 2)
    for k in range(2):
        graphs[k].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        graphs[k % 2].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps

    # algorithmic bytes (every input read once, every output written once)
    D2 = s.D * 2
    ki_row = s.d_I * {"f32": 4, "bf16": 2, "fp8": 1, "fp4": 0.5}[s.idx]
    comp_bytes = (2 * s.T_comp * D2 + s.D * 4 + 2 * (s.T_comp // s.m) * D2 + s.T_comp * s.d_I * 2
                  + (s.T_comp // s.m) * ki_row)
    vis = sum((s.q_pos0 + i + 1) // s.m for i in range(s.Lq))
    n_last = (s.q_pos0 + s.Lq) // s.m
    topk_bytes = (s.B * n_last * s.d_I + s.B * s.Lq * s.H_I * (s.d_I + 4) + 2 * s.B * vis * 4
                  + s.B * s.Lq * s.topk * 4)
    n_w = sum(min(s.W, s.q_pos0 + i + 1) for i in range(s.Lq))
    rows = s.B * (s.Lq * s.topk + n_w)
    io_bytes = s.B * s.Lq * s.topk * 4 + 2 * s.B * s.Lq * s.H * D2 + s.B * s.Lq * s.H * 4
    # rows as gathered, once per query that reads them (most hit L2 / last-level cache) ...
    gathered = rows * 2 * D2 + io_bytes
    # ... and the algorithmic bytes: each distinct compressed entry and raw window row read once
    idx0 = xs[0]["idx"]
    distinct = sum(int(torch.unique(idx0[b][idx0[b] >= 0]).numel()) for b in range(s.B))
    win_rows = s.B * (s.Lq + min(s.W, s.q_pos0 + 1) - 1)
    attn_bytes = (distinct + win_rows) * 2 * D2 + io_bytes
    t_attn = breakdown["sparse_attn"] * 1e-6
    roof = {"bound": "hbm", "achieved": attn_bytes / t_attn / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof.update(traffic=None, kernel="sparse_attn (distinct rows read once; the gathered rows are served by "
                                     "L2 / last-level cache, see gather_gbs)", bytes_per_launch=attn_bytes)
    roof = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()}
    result = {
        "metric": "CSA prefill query-tok/s (chunk 4096 @64K, compress + index_topk + sparse_attn)",
        "value": round(s.Lq / (ms / 1000.0), 1), "unit": "query-tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) caches, queries and indexer inputs in e4m3fn; random-init gate)",
        "config": {"workload": "csa_prefill_chunk4096_ctx64k", "query_chunk": s.Lq, "context": s.q_pos0 + s.Lq,
                   "compressed_entries": s.N_cap, "heads": s.H, "head_dim": s.D,
                   "indexer": "%dx%d %s" % (s.H_I, s.d_I, s.idx), "topk": s.topk, "window": s.W},
        "roofline": roof, "breakdown_us": breakdown,
        "call_gbs": {"compress": round(comp_bytes / (breakdown["compress"] * 1e-6) / 1e9, 1),
                     "index_topk": round(topk_bytes / (breakdown["index_topk"] * 1e-6) / 1e9, 1),
                     "sparse_attn": round(roof["achieved"], 1)},
        "gather_gbs": round(gathered / t_attn / 1e9, 1),
        "timing": "value/ms_per_step: HIP-graph replays of the three calls; breakdown_us: back-to-back launches "
                  "of each call between HIP events; " + SETTLE_NOTE,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _oracle_prefill_baseline(s, xs[0], args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _oracle_prefill_baseline(s, x, seconds):
    """The oracle on the prefill chunk: the chunk's compression once, then
    query by query (indexer scores over the visible entries, top-k, attention
    over the selected rows and the window) until `seconds` of work; the
    compression is charged in proportion to the queries done."""
    import numpy as np
    import torch
    from oracle import attention as oatt, compress as ocmp, formats, indexer as oidx, topk as otopk

    def bf(t_):
        return formats.bf16_to_f64(t_.view(torch.int16).numpy().view(np.uint16))

    def f8(t_):
        return formats.e4m3fn_to_f64(t_.view(torch.uint8).numpy())

    kr_all, vr_all = x["k_raw"][0].cpu(), x["v_raw"][0].cpu()
    kch, vch = x["kraw_chunk"][0].cpu(), x["vraw_chunk"][0].cpu()
    kich = x["kiraw_chunk"][0].cpu()
    w_gate = x["w_gate"].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    _, _, kic = ocmp.compress(bf(kch), bf(vch), w_gate, s.m, s.comp_pos0, x_raw=bf(kich))
    formats.f64_to_e4m3fn(kic)
    t_comp = time.perf_counter() - t0
    kc_all, vc_all = x["k_c"][0].cpu(), x["v_c"][0].cpu()
    ki_all = f8(x["k_i"][0].cpu())
    qi_all, wi_all, q_all = x["q_i"][0].cpu(), x["w_i"][0].cpu(), x["q"][0].cpu()
    sink = x["sink"].cpu().numpy().astype(np.float64)
    K, V = bf(kr_all), bf(vr_all)
    done, spent = 0, 0.0
    while done < s.Lq and (done == 0 or spent < seconds):
        i = done
        t = s.q_pos0 + i
        n = (t + 1) // s.m
        lo = max(0, t - s.W + 1)
        pos = np.arange(lo, t + 1)
        t0 = time.perf_counter()
        sc = oidx.index_scores(f8(qi_all[i]), wi_all[i].numpy().astype(np.float64), ki_all[:n])
        sel = otopk.topk_select(sc, s.topk)
        sel = sel[sel >= 0]
        oatt.attend_one(bf(q_all[i]), t, bf(kc_all[sel]), bf(vc_all[sel]), K[pos - s.raw_pos0], pos,
                        V[pos - s.raw_pos0], sink)
        spent += time.perf_counter() - t0
        done += 1
    spent += t_comp * done / s.Lq
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(blas) if blas else 1
    except Exception:
        cores = 1
    return {"value": round(done / spent, 4), "unit": "query-tok/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d query rows of csa_prefill_chunk4096_ctx64k (plus that share of the chunk's "
                      "compression), %.1f s of oracle work (numpy float64)" % (done, s.Lq, spent)}


def _oracle_bf16_baseline(s, x, seconds):
    """The oracle's indexer scores and bf16-score top-k, query by query, until
    `seconds` of oracle work have run."""
    import numpy as np
    import torch
    from oracle import formats, indexer as oidx, topk as otopk
    ki = x["k_i"][0].cpu().numpy()
    done, spent = 0, 0.0
    while done < s.Lq and (done == 0 or spent < seconds):
        i = done
        qi, wi = x["q_i"][0, i].cpu().numpy(), x["w_i"][0, i].cpu().numpy()
        t0 = time.perf_counter()
        n = (s.q_pos0 + i + 1) // s.m
        sc = oidx.index_scores(formats.e4m3fn_to_f64(qi), wi.astype(np.float64), formats.e4m3fn_to_f64(ki[:n]))
        r = formats.round_bf16(sc)
        otopk.topk_select(r, s.topk)
        spent += time.perf_counter() - t0
        done += 1
    return {"value": round(done / spent, 3), "unit": "query-tok/s", "cores": os.cpu_count(), "kind": "oracle",
            "sample": "%d of %d queries of indexer_bf16_scores_chunk4096_ctx64k_fp8, %.1f s of oracle work "
                      "(numpy float64)" % (done, s.Lq, spent)}


def bench_attn_bwd(args, torch, csa, wl, dev):
    """csa_sparse_attn_bwd on prefill attention shapes: the 2048-token prefill
    (f32, 4 heads x 128, top-64, window 128) and the 4096-token chunk at 64K
    (bf16, top-1024 of 16384 entries, window 128). Selected entries are random
    sorted sets (the gather pattern N(0,1) scores give). Timed with HIP events
    over back-to-back calls (each call: zero the accumulators, the backward
    kernel, the f32 conversion, the sink sum). Algorithmic bytes per call:
    per query the k + W source rows of K and V, q, dout, out and lse read once;
    dq, and dk/dv of every compressed and raw row written once."""
    import numpy as np
    cases = [("prefill_L2048_f32", wl.CFG1), ("chunk4096_ctx64k_bf16", wl.CFG3)]
    res = {}
    for name, s in cases:
        x = wl.make_inputs(s, wl.SEEDS["1" if s is wl.CFG1 else "3"], device=dev)
        rng = np.random.default_rng(7)
        idx = np.full((s.B, s.Lq, s.topk), -1, dtype=np.int32)
        for i in range(s.Lq):
            n = min(s.N_cap, (s.q_pos0 + i + 1) // s.m)
            take = min(n, s.topk)
            idx[0, i, :take] = np.sort(rng.choice(n, size=take, replace=False))
        it = torch.from_numpy(idx).to(dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)
        dout = torch.randn(x["q"].shape, generator=gen, device=dev).to(x["q"].dtype)
        out, lse = csa.sparse_attn(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], s.raw_pos0, s.W, x["sink"],
                                   s.q_pos0)
        wsb = csa.attn_bwd_ws_bytes(s.B, s.Lq, s.q_pos0, 0, s.H, s.D, s.N_cap, s.topk, s.W)
        ws = torch.empty((wsb + 15) // 16 * 4, dtype=torch.float32, device=dev)

        def call():
            return csa.sparse_attn_bwd(x["q"], x["k_c"], x["v_c"], it, x["k_raw"], x["v_raw"], s.raw_pos0, s.W,
                                       x["sink"], s.q_pos0, out, lse, dout, ws=ws)
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        settle(torch, lambda k: call())
        reps = max(3, args.steps // 10)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        us = 1000.0 * e0.elapsed_time(e1) / reps
        kvb = 2 if s.kv == "bf16" else 4
        rows = int((idx >= 0).sum()) + sum(min(s.W, s.q_pos0 + i + 1) for i in range(s.Lq))
        nbytes = (rows * 2 * s.D * kvb + s.B * s.Lq * s.H * (3 * s.D * kvb + 4) + s.B * s.Lq * s.H * s.D * 4
                  + 2 * s.B * (s.N_cap + s.T_raw) * s.D * 4)
        res[name] = {"us": round(us, 1), "queries": s.B * s.Lq, "query_tok_s": round(s.B * s.Lq / (us * 1e-6), 1),
                     "bytes": nbytes, "gbs": round(nbytes / us / 1e3, 1), "source_rows": rows}
        main = (name, s, x, idx, dout)
        del ws
        torch.cuda.empty_cache()
    name, s, x, idx, dout = main
    m = res[name]
    roof = {"bound": "hbm", "achieved": m["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(m["gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "csa_sparse_attn_bwd (all launches of the call)", "bytes_per_launch": m["bytes"]}
    result = {
        "metric": "CSA attention backward query-tok/s (prefill chunk 4096 @64K, top-1024)",
        "value": m["query_tok_s"], "unit": "query-tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(m["us"] / 1000.0, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) q, caches, dout; random sorted selections)",
        "config": {"workload": "csa_attn_bwd_chunk4096_ctx64k", "cases": {c[0]: {"queries": c[1].B * c[1].Lq,
                   "heads": c[1].H, "head_dim": c[1].D, "topk": c[1].topk, "window": c[1].W, "kv": c[1].kv}
                   for c in cases}},
        "roofline": roof, "cases": res,
        "timing": "HIP events over back-to-back calls, " + SETTLE_NOTE,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _oracle_bwd_baseline(s, x, idx, dout, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _oracle_bwd_baseline(s, x, idx, dout, seconds):
    """The oracle's per-query backward (attend_one_bwd) on query rows of the
    workload until `seconds` of oracle work have run."""
    import numpy as np
    import torch
    from oracle import attention_bwd as obwd, formats

    def dec(t_):
        t_ = t_.cpu()
        if t_.dtype == torch.bfloat16:
            return formats.bf16_to_f64(t_.view(torch.int16).numpy().view(np.uint16))
        return t_.numpy().astype(np.float64)
    sink = dec(x["sink"])
    done, spent = 0, 0.0
    while done < s.Lq and (done == 0 or spent < seconds):
        i = s.Lq - 1 - done
        t = s.q_pos0 + i
        sel = idx[0, i][idx[0, i] >= 0]
        lo = max(0, t - s.W + 1)
        pos = np.arange(lo, t + 1)
        rows = torch.from_numpy(sel.astype(np.int64)).to(x["k_c"].device)
        q, kc, vc = dec(x["q"][0, i]), dec(x["k_c"][0][rows]), dec(x["v_c"][0][rows])
        kr, vr = dec(x["k_raw"][0, lo - s.raw_pos0:t + 1 - s.raw_pos0]), dec(x["v_raw"][0, lo - s.raw_pos0:t + 1 - s.raw_pos0])
        do = dec(dout[0, i])
        t0 = time.perf_counter()
        obwd.attend_one_bwd(q, t, kc, vc, kr, pos, vr, sink, do)
        spent += time.perf_counter() - t0
        done += 1
    return {"value": round(done / spent, 3), "unit": "query-tok/s", "cores": os.cpu_count(), "kind": "oracle",
            "sample": "%d of %d query rows of csa_attn_bwd_chunk4096_ctx64k, %.1f s of oracle work (numpy float64)"
                      % (done, s.Lq, spent)}


def copy_ceiling(torch, dev, nbytes=1 << 30, reps=10, settle_s=SETTLE_S):
    """Read+write bandwidth of a plain device copy of nbytes (context for the
    roofline, and the calibration kernel for HBM byte counters)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    settle(torch, lambda k: dst.copy_(src), settle_s)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1000.0 / reps
    del src, dst
    return round(2 * nbytes / sec / 1e9, 1)


def prefill_indexer_mfma(torch, csa, wl, dev, reps=20, warmup=10):
    """The second half of the headline metric: the fp8 indexer QK of a
    4096-token prefill chunk at 64K context with 64 heads x 128 dims (the
    MFMA-bound reading of that workload), as a fraction of the fp8 MFMA peak.
    Mean of `reps` back-to-back launches between HIP events on the launch
    stream, after `warmup` launches; two input sets alternate."""
    s = wl.CFG3M
    xs = []
    for sd in (wl.SEEDS["3M"], 1000 + wl.SEEDS["3M"]):
        gen = torch.Generator(device=dev)
        gen.manual_seed(sd)
        x = wl.indexer_inputs(s, gen, dev)
        x["scores"] = torch.empty((s.B, s.Lq, s.N_cap), dtype=torch.float32, device=dev)
        xs.append(x)

    def launch(x):
        csa.index_scores(x["q_i"], x["w_i"], x["k_i"], s.q_pos0, s.m, s.idx, x["q_i_scale"], x["k_i_scale"],
                         out=x["scores"])
    for k in range(warmup):
        launch(xs[k % 2])
    settle(torch, lambda k: launch(xs[k % 2]))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(reps):
        launch(xs[k % 2])
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / reps
    fl = index_qk_flops(s)
    tf = fl / (us * 1e-6) / 1e12
    del xs
    return {"workload": s.name, "kernel": "index_qk_prefill (fp8 64x128)", "us": round(us, 2),
            "flops_per_launch": fl, "achieved": round(tf, 1), "peak": MFMA_PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
            "frac": round(tf / MFMA_PEAK_TFLOPS["fp8"], 4),
            "timing": "mean of %d back-to-back launches after %d warmup launches, %s" % (reps, warmup, SETTLE_NOTE)}


# ------------------------------------------------------------- CPU baseline
def _oracle_query(s, x, b):
    """Oracle seconds for query token b of workload s; copying the input rows it
    reads from the GPU to the host is not timed."""
    import numpy as np
    import torch
    from oracle import attention as oatt, formats, indexer as oidx, topk as otopk

    def bf(t):
        return formats.bf16_to_f64(t.view(torch.int16).numpy().view(np.uint16))

    t = s.q_pos0
    n = (t + 1) // s.m
    lo = max(0, t - s.W + 1)
    pos = np.arange(lo, t + 1)
    q = x["q"][b].cpu()
    sink = x["sink"].cpu().numpy().astype(np.float64)
    spent = 0.0
    if s.H_I:
        qi, wi = x["q_i"][b].cpu(), x["w_i"][b].cpu()
        ki = x["k_i"][b][:n].cpu()
        qs = x["q_i_scale"][b].cpu() if x["q_i_scale"] is not None else None
        ks = x["k_i_scale"][b][:n].cpu() if x["k_i_scale"] is not None else None
        t0 = time.perf_counter()
        if s.idx == "fp4":
            qd, kd = formats.mxfp4_to_f64(qi[0].numpy(), qs[0].numpy()), formats.mxfp4_to_f64(ki.numpy(), ks.numpy())
        else:
            qd, kd = bf(qi[0]), bf(ki)
        sc = oidx.index_scores(qd, wi[0].numpy().astype(np.float64), kd)
        sel = otopk.topk_select(sc, s.topk)
        sel = sel[sel >= 0]
        spent += time.perf_counter() - t0
        rows = torch.from_numpy(sel).to(x["k_c"].device)
        kc, vc = x["k_c"][b][rows].cpu(), x["v_c"][b][rows].cpu()
    else:
        kc, vc = x["k_c"][b][:n].cpu(), x["v_c"][b][:n].cpu()
    kr = x["k_raw"][b][pos[0] - s.raw_pos0:pos[-1] + 1 - s.raw_pos0].cpu()
    vr = x["v_raw"][b][pos[0] - s.raw_pos0:pos[-1] + 1 - s.raw_pos0].cpu()
    t0 = time.perf_counter()
    oatt.attend_one(bf(q[0]), t, bf(kc), bf(vc), bf(kr), pos, bf(vr), sink)
    spent += time.perf_counter() - t0
    return spent


def _oracle_state_query(s, x, b, t):
    """Oracle seconds for one decode step of sequence b at position t with the
    state cache: the token enters the ring and, when it completes a block, the
    block is compressed (the oracle's state-cache steps), then indexer,
    top-k and attention with the window read from the ring. Copying the rows
    it reads from the GPU is not timed."""
    import numpy as np
    import torch
    from oracle import attention as oatt, compress as ocmp, formats, indexer as oidx, topk as otopk

    def bf(t_):
        return formats.bf16_to_f64(t_.view(torch.int16).numpy().view(np.uint16))

    R = x["k_raw"].shape[1]
    n = (t + 1) // s.m
    kr, vr, xr = x["k_raw"][b].cpu(), x["v_raw"][b].cpu(), x["ki_ring"][b].cpu()
    kn, vn, xn = x["k_new"][b].cpu(), x["v_new"][b].cpu(), x["ki_new"][b].cpu()
    w_gate = x["w_gate"].cpu().numpy().astype(np.float64)
    qi, wi, ki = x["q_i"][b].cpu(), x["w_i"][b].cpu(), x["k_i"][b][:n].cpu()
    q, sink = x["q"][b].cpu(), x["sink"].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    K, V, X = bf(kr), bf(vr), bf(xr)
    K[t % R], V[t % R], X[t % R] = bf(kn), bf(vn), bf(xn)
    if (t + 1) % s.m == 0:
        blk = np.arange(t - s.m + 1, t + 1) % R
        ocmp.compress(K[blk], V[blk], w_gate, s.m, pos0=t - s.m + 1, x_raw=X[blk])
    sc = oidx.index_scores(bf(qi[0]), wi[0].numpy().astype(np.float64), bf(ki))
    sel = otopk.topk_select(sc, s.topk)
    sel = sel[sel >= 0]
    spent = time.perf_counter() - t0
    rows = torch.from_numpy(sel).to(x["k_c"].device)
    kc, vc = x["k_c"][b][rows].cpu(), x["v_c"][b][rows].cpu()
    t0 = time.perf_counter()
    pos = np.arange(max(0, t - s.W + 1), t + 1)
    oatt.attend_one(bf(q[0]), t, bf(kc), bf(vc), K[pos % R], pos, V[pos % R], sink)
    return spent + time.perf_counter() - t0


def _blas_cores():
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(blas) if blas else 1
    except Exception:
        return 1


def _cpu_model():
    cpu = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return cpu


def _sample(parts, seconds, query_fn):
    """Oracle query tokens until `seconds` of oracle work: the batch's tokens
    in order, cycled when one pass takes less. Returns (tokens, seconds)."""
    B = parts[0][0].B
    done, spent = 0, 0.0
    while done == 0 or spent < seconds:
        for s, x in parts:
            spent += query_fn(s, x, done % B) if query_fn else _oracle_query(s, x, done % B)
        done += 1
    return done, spent


def cpu_baseline(wl_name, parts, seconds, query_fn=None):
    """Time the CPU oracle, as it stands, on whole query tokens of the same
    workload (every layer of it) until `seconds` of oracle work have run:
    once with the BLAS threads numpy starts with (all host cores), once with
    one thread."""
    cores = _blas_cores()
    B = parts[0][0].B
    done, spent = _sample(parts, seconds, query_fn)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            d1, s1 = _sample(parts, seconds, query_fn)
        one = {"value": round(d1 / s1, 4), "cores": 1,
               "sample": "%d query tokens (the batch's %d in order, cycled), %.1f s of oracle work" % (d1, B, s1)}
    except ImportError:
        pass
    return {"value": round(done / spent, 4), "unit": "query-tok/s", "cores": cores, "kind": "oracle",
            "sample": "%d query tokens (the batch's %d in order, cycled) of %s, %.1f s of oracle work (numpy float64, BLAS threads %d; "
                      "host has %d CPUs: %s)" % (done, B, wl_name, spent, cores, os.cpu_count(), _cpu_model()),
            "one_thread": one}


# -------------------------------------------------------------------- main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build measures one GPU's share of the work "
              "(--gpus %d, WORLD_SIZE %d requested)." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_attention_16_amd as csa
    from long_context_attention_16_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    csa.lib()

    if args.copy_only:
        print(json.dumps({"copy_gbs": copy_ceiling(torch, dev, settle_s=0.0), "bytes_per_copy": 2 * (1 << 30)}),
              flush=True)
        return

    W = args.workload
    if W == "compress":
        bench_compress(args, torch, csa, dev)
        return
    if W == "csa_decode_state":
        bench_state_decode(args, torch, csa, wl, dev)
        return
    if W == "indexer_bf16_scores":
        bench_bf16_scores(args, torch, csa, wl, dev)
        return
    if W == "csa_attn_bwd":
        bench_attn_bwd(args, torch, csa, wl, dev)
        return
    if W == "csa_prefill":
        bench_prefill(args, torch, csa, wl, dev)
        return
    if W == "csa_decode":
        shapes = [("", wl.CFG2)]
    elif W == "hca_decode":
        shapes = [("", wl.CFG4)]
    elif W == "pair_1m":
        shapes = [("csa.", wl.CFG5_CSA), ("hca.", wl.CFG5_HCA)]
    else:
        shapes = [("", wl.CFG3M)]

    sets = []
    for prefix, s in shapes:
        base = {"csa_decode": "2", "hca_decode": "4", "indexer_fp8_prefill": "3M"}.get(W)
        base = base or ("5csa" if s.H_I else "5hca")
        seeds = [wl.SEEDS[base], 1000 + wl.SEEDS[base]]
        if s.H_I and W != "indexer_fp8_prefill":
            sets.append(csa_decode_setup(torch, csa, wl, s, seeds, dev))
        elif s.H_I:
            xs = []
            for sd in seeds:
                gen = torch.Generator(device=dev)
                gen.manual_seed(sd)
                x = wl.indexer_inputs(s, gen, dev)
                x["scores"] = torch.empty((s.B, s.Lq, s.N_cap), dtype=torch.float32, device=dev)
                xs.append(x)
            sets.append(xs)
        else:
            sets.append(hca_setup(torch, csa, wl, s, seeds, dev))
    torch.cuda.synchronize()

    labels = []
    for prefix, s in shapes:
        if W == "indexer_fp8_prefill":
            labels += [prefix + "index_qk"]
        elif s.H_I and fused(s):
            labels += [prefix + "index_cand", prefix + "topk_merge", prefix + "sparse_attn"]
        elif s.H_I:
            labels += [prefix + "index_qk", prefix + "topk", prefix + "sparse_attn"]
        else:
            labels += [prefix + "hca_attn"]

    def launch(label, x, s):
        """One library call of the step (kernel(s) named by label)."""
        kind = label.split(".")[-1]
        if kind == "index_qk":
            csa.index_scores(x["q_i"], x["w_i"], x["k_i"], s.q_pos0, s.m, s.idx, x["q_i_scale"], x["k_i_scale"],
                             out=x["scores"])
        elif kind == "index_cand":
            csa.index_candidates(x["q_i"], x["w_i"], x["k_i"], s.topk, s.q_pos0, s.m, s.idx, x["q_i_scale"],
                                 x["k_i_scale"], cand=x["cand"])
        elif kind == "topk_merge":
            csa.topk_merge(x["cand"], s.B, s.Lq, s.topk, s.q_pos0, s.m, out=x["idx"])
        elif kind == "topk":
            csa.topk(x["scores"], s.topk, s.q_pos0, s.m, out=x["idx"], ws=x["topk_ws"])
        elif kind == "sparse_attn":
            csa.sparse_attn(x["q"], x["k_c"], x["v_c"], x["idx"], x["k_raw"], x["v_raw"], s.raw_pos0, s.W,
                            x["sink"], s.q_pos0, ws=x["ws"], out=x["out"], lse=x["lse"])
        else:
            csa.hca_attn(x["q"], x["k_c"], x["v_c"], s.m, x["k_raw"], x["v_raw"], s.raw_pos0, s.W, x["sink"],
                         s.q_pos0, ws=x["ws"], out=x["out"], lse=x["lse"])

    def step(k):
        for (prefix, s), xs in zip(shapes, sets):
            x = xs[k % len(xs)]
            for l in labels:
                if l.startswith(prefix) and (prefix or "." not in l):
                    launch(l, x, s)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # The timed steps: one HIP graph per input set (the library's kernels are
    # captured on torch's capture stream; they use no memsets), replayed
    # alternately so consecutive steps read different inputs. Captured first,
    # so that the clock settle below runs the step itself and no idle gap
    # (the capture) separates it from the timed regions.
    graphs = []
    for k in range(2):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            step(k)
        graphs.append(gph)
    settle(torch, lambda k: graphs[k % 2].replay())

    # Per-kernel average durations: back-to-back launches of each call (both
    # input sets alternating) between HIP events on the launch stream.
    breakdown = {}
    for (prefix, s), xs in zip(shapes, sets):
        for l in labels:
            if not (l.startswith(prefix) and (prefix or "." not in l)):
                continue
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for k in range(args.steps):
                launch(l, xs[k % len(xs)], s)
            e1.record()
            torch.cuda.synchronize()
            breakdown[l] = round(1000.0 * e0.elapsed_time(e1) / args.steps, 2)

    for k in range(args.warmup):
        graphs[k % 2].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        graphs[k % 2].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1000.0 / args.steps

    main_shape = shapes[0][1]
    queries = main_shape.B * main_shape.Lq
    value = queries / (ms / 1000.0)
    if W == "csa_decode":
        metric, unit = "CSA decode query-tok/s @128K ctx", "query-tok/s"
        dom = "index_cand"
        dom_bytes = index_cand_bytes(main_shape)
        roof = {"bound": "hbm", "achieved": dom_bytes / (breakdown[dom] * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
        cfg = {"workload": main_shape.name, "batch": main_shape.B, "context": main_shape.q_pos0 + 1,
               "compressed_entries": main_shape.N_cap, "heads": main_shape.H, "head_dim": main_shape.D,
               "indexer": "%dx%d %s" % (main_shape.H_I, main_shape.d_I, main_shape.idx),
               "topk": main_shape.topk, "window": main_shape.W}
        step_bytes = index_cand_bytes(main_shape) + topk_merge_bytes(main_shape) + sparse_attn_bytes(main_shape)
    elif W == "hca_decode":
        metric, unit = "HCA decode query-tok/s @1M ctx", "query-tok/s"
        dom = "hca_attn"
        dom_bytes = hca_bytes(main_shape)
        roof = {"bound": "hbm", "achieved": dom_bytes / (breakdown[dom] * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
        cfg = {"workload": main_shape.name, "batch": main_shape.B, "context": main_shape.q_pos0 + 1,
               "compressed_entries": main_shape.N_cap, "m": main_shape.m, "heads": main_shape.H,
               "head_dim": main_shape.D, "window": main_shape.W}
        step_bytes = dom_bytes
    elif W == "pair_1m":
        metric, unit = "CSA+HCA layer-pair decode query-tok/s @1M ctx", "query-tok/s"
        # the CSA half's indexer runs fused (k = 1024: 4096-entry chunks)
        dom = "csa.index_cand" if fused(main_shape) else "csa.index_qk"
        dom_bytes = index_cand_bytes(main_shape) if fused(main_shape) else index_qk_bytes(main_shape)
        roof = {"bound": "hbm", "achieved": dom_bytes / (breakdown[dom] * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
        cfg = {"workload": "csa_hca_pair_1m_b8", "batch": main_shape.B, "context": main_shape.q_pos0 + 1,
               "csa_entries": main_shape.N_cap, "hca_entries": wl.CFG5_HCA.N_cap,
               "indexer": "%dx%d mxfp4" % (main_shape.H_I, main_shape.d_I), "topk": main_shape.topk,
               "heads": main_shape.H, "head_dim": main_shape.D, "window": main_shape.W}
        sel_bytes = (index_cand_bytes(main_shape) + topk_merge_bytes(main_shape) if fused(main_shape)
                     else index_qk_bytes(main_shape) + topk_bytes(main_shape))
        step_bytes = sel_bytes + sparse_attn_bytes(main_shape) + hca_bytes(wl.CFG5_HCA)
    else:
        metric, unit = "indexer fp8 prefill query-tok/s @64K ctx", "query-tok/s"
        dom = "index_qk"
        fl = index_qk_flops(main_shape)
        dom_bytes = index_qk_bytes(main_shape)
        roof = {"bound": "mfma", "achieved": fl / (breakdown[dom] * 1e-6) / 1e12,
                "peak": MFMA_PEAK_TFLOPS["fp8"], "unit": "TFLOP/s"}
        cfg = {"workload": main_shape.name, "batch": main_shape.B, "query_chunk": main_shape.Lq,
               "context": main_shape.q_pos0 + main_shape.Lq, "compressed_entries": main_shape.N_cap,
               "indexer": "%dx%d fp8" % (main_shape.H_I, main_shape.d_I)}
        step_bytes = index_qk_bytes(main_shape)
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(W, dom)
    roof["kernel"] = dom
    roof["bytes_per_launch"] = dom_bytes
    roof["scope"] = "dominant kernel only (the whole step: step_hbm_gbs, step_frac)"
    roof = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()}

    result = {
        "metric": metric, "value": round(value, 1), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": main_shape.kv if W != "indexer_fp8_prefill" else "fp8",
        "data": "synthetic (seeded N(0,1) caches and queries, random-init indexer; no weights or datasets)",
        "config": cfg, "roofline": roof,
        "breakdown_us": breakdown,
        "timing": "value/ms_per_step: HIP-graph replays of the whole step; breakdown_us and roofline: "
                  "back-to-back launches of each call between HIP events; " + SETTLE_NOTE,
        "step_hbm_gbs": round(step_bytes / (ms / 1000.0) / 1e9, 1),
        "step_frac": round(step_bytes / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        "copy_ceiling_gbs": copy_ceiling(torch, dev),
    }
    if W == "csa_decode":
        result["indexer_mfma"] = prefill_indexer_mfma(torch, csa, wl, dev)
    if args.no_cpu_baseline:
        result["cpu_baseline"] = None
    elif W == "indexer_fp8_prefill":
        result["cpu_baseline"] = _oracle_prefill_indexer_baseline(main_shape, sets[0][0], args.cpu_seconds)
    else:
        parts = [(s, xs[0]) for (prefix, s), xs in zip(shapes, sets)]
        result["cpu_baseline"] = cpu_baseline(cfg["workload"], parts, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
