#!/usr/bin/env python3
"""Benchmark of the CSA/HCA attention forward on one MI355X.

Headline workload (the metric's "1M-ctx decode"): one decode step of an
alternating CSA + HCA layer pair at a 1,048,576-token context, batch 8:
  CSA: indexer over 262,144 compressed entries with fp4 (e2m1, 1x32 E8M0)
       keys, 64 indexer heads x 128, top-k 1024, then sparse attention over
       the 1024 selected entries + the 128-token window + sink, 128 heads;
  HCA: dense attention over 8,192 compressed entries + window + sink.
A step = indexer_topk + sparse_attn_fwd + dense_compressed_attn_fwd on
caches already resident in HBM, replayed as a HIP graph. Four independent
copies of the caches are rotated so the 256 MB Infinity Cache cannot serve a
step from the previous one. ``value`` = queries/s = B / step time.

Also reported: the step's algorithmic HBM bytes / step time, the dominant
kernel's roofline fraction (the indexer's score stage: back-to-back launches
in one HIP graph timed with HIP events on the stream they run on), the
selection recall of the fp4 keys against float32, the CPU oracle timed on a
bounded sample, and extra workloads (the same decode pair at batches 16, 32
and 64, CSA decode at 262k context, cache appends, prefill and backward
TFLOP/s, projections) under "extras".

Usage: python bench.py [--steps K] [--warmup W]
                       [--extras decode_batches,decode4,decode_bf16,decode_append,prefill_csa,prefill_hca,
                                 prefill_chunk,bwd_csa,bwd_hca,proj|none]
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

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0
METRIC = "CSA/HCA attn queries/sec + achieved HBM TB/s at 1M-ctx decode; prefill TFLOP/s"
# The pages' model-level claims (no hardware stated; context, not a target):
# per-token inference FLOPs and KV-cache size relative to DeepSeek-V3.2 at a
# 1M-token context.
PAGES_CLAIMS = {
    "V4-Pro_vs_V3.2_at_1M_ctx": {"flops": 0.27, "kv_cache": 0.10},
    "V4-Flash_vs_V3.2_at_1M_ctx": {"flops": 0.10, "kv_cache": 0.07},
    "source": "cf-1.com write-up §1; yfxerp.com write-up 'DeepSeek-V4 原理拆解' §1",
    "hardware": "not stated",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def recorded_traffic(kernel: str, source: str):
    """HBM bytes per launch (read + written) of `kernel` from the committed
    rocprofv3 counter summary, or None if the kernel's source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "csa_hca_decode_1m_hbm_counters.md")
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(os.path.join(ROOT, source), "rb").read()).hexdigest()[:16]
    for line in open(path):
        if line.startswith("TRAFFIC ") and f"kernel={kernel} " in line:
            kv = dict(f.split("=", 1) for f in line.split()[1:])
            if kv.get("src_sha256_16") == sha:
                return int(kv["read_bytes"]) + int(kv["write_bytes"])
    return None


# ----------------------------------------------------------------------------- decode workloads

def decode_workload(torch, C, syn, name, B, L, H, H_I, d_I, k, fmt, hca, copies, wid, host_sample=True,
                    bf16_scores=False):
    """Build the caches (copies of them) and one-step closures for a decode workload."""
    dev = "cuda"
    N = L // 4
    NH = L // 128
    bf = torch.bfloat16
    s = 1000 * wid
    st = {"B": B, "L": L, "N": N, "NH": NH, "H": H, "H_I": H_I, "d_I": d_I, "k": k, "fmt": fmt}
    # keys: generate once in float32 on the device, quantise with the library
    ki32 = syn.normal_device(s + 2, (B, N, d_I), dev)
    codes, scales = C.csa_quantize_rows(ki32, fmt)
    if host_sample:
        st["ki_host_rows"] = ki32[: min(B, 8)].cpu()   # for the CPU baseline sample
    st["ki32_rows"] = ki32[:2].clone()                 # unquantised keys of two sequences (recall of the format)
    del ki32
    kv = syn.normal_device(s + 1, (B, N, 128), dev, bf)
    if host_sample:
        st["kv_host"] = kv[: min(B, 8)].float().cpu()
    st["codes"], st["scales"], st["kv"] = [codes], [scales], [kv]
    for _ in range(copies - 1):
        st["codes"].append(codes.clone())
        st["scales"].append(scales.clone())
        st["kv"].append(kv.clone())
    st["x_win"] = syn.normal_device(s + 3, (B, 128, 128), dev, bf)
    st["q"] = syn.normal_device(s + 4, (B, 1, H, 128), dev, bf, scale=1 / np.sqrt(128))
    qi32 = syn.normal_device(s + 5, (B, 1, H_I, d_I), dev)
    st["qi32"] = qi32
    st["qi"], st["qs"] = C.csa_quantize_rows(qi32, fmt)
    st["w"] = syn.uniform_device(s + 6, (B, 1, H_I), dev)
    st["sink"] = syn.normal_device(s + 7, (H,), dev)
    st["q_pos"] = torch.full((B, 1), L, dtype=torch.int32, device=dev)
    st["win_start"] = torch.full((B,), L - 127, dtype=torch.int32, device=dev)
    st["idx"] = torch.empty(B, 1, k, dtype=torch.int32, device=dev)
    st["out"] = torch.empty(B, 1, H, 128, dtype=bf, device=dev)
    st["ws_idx"] = torch.empty(C.indexer_topk_workspace_size(B, 1, N, H_I, d_I, k, fmt, bf16_scores),
                               dtype=torch.uint8, device=dev)
    st["ws_sp"] = torch.empty(max(1, C.sparse_attn_workspace_size(B, 1, H, 128, k, 128)), dtype=torch.uint8, device=dev)
    bytes_idx = B * N * (d_I // 2 + d_I // 32 if fmt == "fp4" else d_I + 4) + B * H_I * (d_I + 8)
    bytes_sp = B * (k + 128) * 256 + 2 * B * H * 256 + B * k * 4
    st["bytes_index_score"] = bytes_idx
    st["bytes"] = bytes_idx + bytes_sp
    if hca:
        kvh = syn.normal_device(s + 11, (B, NH, 128), dev, bf)
        if host_sample:
            st["kvh_host"] = kvh[: min(B, 8)].float().cpu()
        st["kvh"] = [kvh] + [kvh.clone() for _ in range(copies - 1)]
        st["xh"] = syn.normal_device(s + 12, (B, 128, 128), dev, bf)
        st["qh"] = syn.normal_device(s + 13, (B, 1, H, 128), dev, bf, scale=1 / np.sqrt(128))
        st["sinkh"] = syn.normal_device(s + 14, (H,), dev)
        st["outh"] = torch.empty(B, 1, H, 128, dtype=bf, device=dev)
        st["ws_dn"] = torch.empty(max(1, C.dense_attn_workspace_size(B, 1, NH, H, 128, 128)), dtype=torch.uint8,
                                  device=dev)
        st["bytes"] += B * (NH + 128) * 256 + 2 * B * H * 256

    def step(c):
        C.indexer_topk(st["qi"], st["qs"], st["w"], st["codes"][c], st["scales"][c], fmt, st["q_pos"], 4, k, d_I,
                       ws=st["ws_idx"], idx_out=st["idx"], bf16_scores=bf16_scores)
        C.sparse_attn_fwd(st["q"], st["kv"][c], st["idx"], st["x_win"], st["win_start"], st["sink"], st["q_pos"],
                          128, 1.0, ws=st["ws_sp"], out=st["out"])
        if hca:
            C.dense_compressed_attn_fwd(st["qh"], st["kvh"][c], st["xh"], st["win_start"], st["sinkh"],
                                        st["q_pos"], 128, 128, 1.0, ws=st["ws_dn"], out=st["outh"])
    st["step"] = step
    st["name"] = name
    st["hca"] = hca
    return st


def decode_batches(torch, C, syn, steps, warmup):
    """The 1M-context decode pair (the headline step) at larger batches, two
    rotated cache copies (every copy's step reads more than the 256 MB
    Infinity Cache holds): the step's fixed per-kernel latencies amortise over
    more sequences, and its HBM rate approaches the score stage's."""
    rows = []
    for B in (16, 32, 64):
        st = decode_workload(torch, C, syn, f"csa_hca_decode_pair_1m_ctx_b{B}", B=B, L=1 << 20, H=128, H_I=64,
                             d_I=128, k=1024, fmt="fp4", hca=True, copies=2, wid=7, host_sample=False)
        del st["ki32_rows"]
        torch.cuda.synchronize()
        ms, _ = time_graphs(torch, st, 2, steps, warmup)
        gbs = st["bytes"] / (ms * 1e-3) / 1e9
        rows.append({"batch": B, "us_per_step": round(ms * 1e3, 1), "queries_per_s": round(B / (ms * 1e-3), 1),
                     "step_bytes": st["bytes"], "hbm_gb_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
        log(f"[bench] decode pair 1M, batch {B}: {rows[-1]}")
        del st
        torch.cuda.empty_cache()
    return {"workload": "csa_hca_decode_pair_1m_ctx_batches", "rows": rows, "cache_copies": 2,
            "timing": "hip graph replay"}


def time_graphs(torch, st, copies, steps, warmup, use_graph=True):
    """Capture one graph per cache copy; replay round-robin. Returns ms/step."""
    step = st["step"]
    for c in range(copies):
        step(c)
    torch.cuda.synchronize()
    if use_graph:
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(copies):
                step(c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        run = lambda i: graphs[i % copies].replay()
    else:
        run = lambda i: step(i % copies)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall


def kernel_times(torch, C, st, copies, steps, kernel):
    """Average duration of one library kernel over `steps` eager steps (HIP events
    recorded by the library on the stream the kernel runs on)."""
    C.kernel_timer_start(kernel, steps)
    for i in range(steps):
        st["step"](i % copies)
    torch.cuda.synchronize()
    t = C.kernel_timer_read(steps)
    return float(np.mean(t)) if t else None


def score_kernel_us(torch, C, st, launches=48, reps=5):
    """Average duration of the indexer score kernel alone: `launches`
    back-to-back indexer_scores calls (the score stage of the step's
    indexer_topk, without the selection's candidate lists), rotating over the
    cache copies like the step, captured in one HIP graph and replayed `reps`
    times between HIP events on the stream the kernels run on; returns
    microseconds per launch. (The library's per-launch event timer adds the
    launch itself to every sample.)"""
    out = torch.empty(st["B"], 1, st["N"], dtype=torch.float32, device="cuda")
    copies = len(st["codes"])
    call = lambda c: C.indexer_scores(st["qi"], st["qs"], st["w"], st["codes"][c], st["scales"][c], st["fmt"],
                                      st["q_pos"], 4, st["d_I"], out=out)
    for c in range(copies):
        call(c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            call(i % copies)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * launches)


def format_recall(torch, C, st):
    """Recall of the quantised indexer keys' selection against the selection on
    the same keys and queries in float32 (the format's own loss), over two
    sequences: |quantised top-k & float32 top-k| / k per row."""
    B2 = st["ki32_rows"].shape[0]
    idx_q = C.indexer_topk(st["qi"][:B2], st["qs"][:B2], st["w"][:B2], st["codes"][0][:B2], st["scales"][0][:B2],
                           st["fmt"], st["q_pos"][:B2], 4, st["k"], st["d_I"])
    idx_f = C.indexer_topk(st["qi32"][:B2].contiguous(), None, st["w"][:B2], st["ki32_rows"], None, "f32",
                           st["q_pos"][:B2], 4, st["k"], st["d_I"])
    a, b = idx_q.cpu().numpy().reshape(B2, -1), idx_f.cpu().numpy().reshape(B2, -1)
    return [round(len(set(a[i]) & set(b[i])) / st["k"], 4) for i in range(B2)]


def cpu_baseline_decode(O, st, seconds):
    """The oracle on the host: the whole decode step (indexer scores, top-k,
    sparse attention, and the HCA layer's dense attention), one sequence at a
    time, repeated over the sampled sequences until about `seconds` of CPU
    time are spent. Inputs (dequantised keys) are prepared outside the timer."""
    B, N, k, fmt = st["B"], st["N"], st["k"], st["fmt"]
    L = st["L"]
    quant, deq = ((O.quant_mxfp4_rows, O.dequant_mxfp4_rows) if fmt == "fp4" else (O.quant_fp8_rows, O.dequant_fp8_rows))
    qi = st["qi32"].cpu().numpy()
    w = st["w"].cpu().numpy()
    q = st["q"].float().cpu().numpy()
    xw = st["x_win"].float().cpu().numpy()
    sink = st["sink"].cpu().numpy()
    if st["hca"]:
        qh = st["qh"].float().cpu().numpy()
        xh = st["xh"].float().cpu().numpy()
        sinkh = st["sinkh"].cpu().numpy()
    nsample = min(2, st["ki_host_rows"].shape[0])
    prep = []
    for b in range(nsample):
        kd = deq(*quant(st["ki_host_rows"][b].numpy()))
        qd = deq(*quant(qi[b]))
        kvb = st["kv_host"][b].numpy()
        kvh = st["kvh_host"][b].numpy() if st["hca"] else None
        prep.append((b, kd, qd, kvb, kvh))
    done, spent = 0, 0.0
    while spent < seconds:
        b, kd, qd, kvb, kvh = prep[done % nsample]
        t0 = time.perf_counter()
        s = O.indexer_scores(qd, w[b], kd, [L], 4)
        idx = O.topk_select(s, O.visible_entries([L], 4, N), k)
        O.sparse_attn(q[b], kvb, idx, xw[b], L - 127, sink, [L], 128)
        if st["hca"]:
            O.dense_attn(qh[b], kvh, xh[b], L - 127, sinkh, [L], 128, 128)
        spent += time.perf_counter() - t0
        done += 1
    return done, spent


def run_decode(torch, C, syn, O, args, which):
    if which in ("pair1m", "pair1m_bf16"):
        bf = which == "pair1m_bf16"
        st = decode_workload(torch, C, syn, "csa_hca_decode_pair_1m_ctx" + ("_bf16_scores" if bf else ""), B=8,
                             L=1 << 20, H=128, H_I=64, d_I=128, k=1024, fmt="fp4", hca=True, copies=args.copies,
                             wid=5, host_sample=not args.no_cpu_baseline and not bf, bf16_scores=bf)
    else:
        st = decode_workload(torch, C, syn, "csa_decode_262k_ctx", B=32, L=1 << 18, H=128, H_I=64, d_I=128,
                             k=1024, fmt="fp8", hca=False, copies=args.copies, wid=4, host_sample=False)
    torch.cuda.synchronize()
    log(f"[bench] {st['name']}: setup done")
    ms, wall = time_graphs(torch, st, args.copies, args.steps, args.warmup, use_graph=not args.eager)
    log(f"[bench] {st['name']}: {ms * 1e3:.1f} us/step (graph), wall {wall * 1e3:.1f} us/step")
    kt = {}
    for kname in ("index_score", "topk", "sparse_attn", "attn_merge", "dense_attn"):
        if kname == "dense_attn" and not st["hca"]:
            continue
        kt[kname] = kernel_times(torch, C, st, args.copies, args.steps, kname)
    log(f"[bench] {st['name']}: kernel us {({k_: (None if v is None else round(v * 1e3, 1)) for k_, v in kt.items()})}")
    st["score_us"] = score_kernel_us(torch, C, st)
    st["recall"] = format_recall(torch, C, st)
    del st["ki32_rows"]
    log(f"[bench] {st['name']}: score kernel alone {st['score_us']:.2f} us/launch, "
        f"{st['fmt']} recall vs float32 {st['recall']}")
    return st, ms, wall, kt


# ----------------------------------------------------------------------------- prefill workloads

def time_ops(torch, ops, iters, warmup=1):
    """Median device time (ms) of each named op over `iters` runs; ops run on the
    current stream, which is the stream the library launches on."""
    for _ in range(warmup):
        for _, f in ops:
            f()
    torch.cuda.synchronize()
    res = {name: [] for name, _ in ops}
    for _ in range(iters):
        for name, f in ops:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            res[name].append(e0.elapsed_time(e1))
    return {k: float(np.median(v)) for k, v in res.items()}


def call_kernel_ms(torch, C, fn, kernel, max_launches=512):
    """Sum of the device times of every launch of one library kernel in one call of fn."""
    C.kernel_timer_start(kernel, max_launches)
    fn()
    torch.cuda.synchronize()
    t = C.kernel_timer_read(max_launches)   # also stops the timer
    return float(np.sum(t)) if t else None


def attn_flops(n_keys, H, d=128):
    """QK and PV: 4 flops per (query, key, head, channel)."""
    return float(np.sum(n_keys, dtype=np.float64)) * H * d * 4


def index_flops(n_vis, H_I, d_I):
    return float(np.sum(n_vis, dtype=np.float64)) * H_I * d_I * 2


def bf16_score_variant(torch, C, iters, call, ws_bytes):
    """Indexer with bfloat16 index scores on the same operands: op time and the
    score / top-k kernel split (ms). Not part of the layer time."""
    ws_b = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")
    fn = lambda: call(ws_b)
    t = time_ops(torch, [("indexer_topk_bf16_scores", fn)], iters)["indexer_topk_bf16_scores"]
    split = {kn: call_kernel_ms(torch, C, fn, kn) for kn in ("index_score", "topk")}
    return {"ms": round(t, 4), "split_ms": {kn: (None if v is None else round(v, 4)) for kn, v in split.items()}}


def prefill_csa(torch, C, syn, iters):
    """Single CSA layer prefill, bf16, T = 65,536: compress (KV and fp8 indexer
    keys), indexer top-512 over 16,384 entries (64 heads x 128, fp8), sparse
    attention with 64 heads, window 128, sink."""
    dev, bf = "cuda", torch.bfloat16
    T, H, H_I, d_I, k, W = 65536, 64, 64, 128, 512, 128
    s = 2000
    c = {n: syn.normal_device(s + i, (1, T, 128), dev, bf) for i, n in enumerate(["c_a", "c_b", "z_a", "z_b"])}
    ci = {n: syn.normal_device(s + 10 + i, (1, T, d_I), dev, bf) for i, n in enumerate(["a", "b", "za", "zb"])}
    q = syn.normal_device(s + 20, (1, T, H, 128), dev, bf, scale=1 / np.sqrt(128))
    qi32 = syn.normal_device(s + 21, (1, T, H_I, d_I), dev)
    qi, qs = C.csa_quantize_rows(qi32, "fp8")
    del qi32
    w = syn.uniform_device(s + 22, (1, T, H_I), dev)
    sink = syn.normal_device(s + 23, (H,), dev)
    q_pos = torch.arange(T, dtype=torch.int32, device=dev)[None]
    win_start = torch.zeros(1, dtype=torch.int32, device=dev)
    N = T // 4
    st = {}
    st["E"] = C.csa_compress(c["c_a"], c["c_b"], c["z_a"], c["z_b"], 4)
    st["KI"] = C.csa_compress(ci["a"], ci["b"], ci["za"], ci["zb"], 4, out_fmt="fp8")
    st["idx"] = torch.empty(1, T, k, dtype=torch.int32, device=dev)
    ws_i = torch.empty(C.indexer_topk_workspace_size(1, T, N, H_I, d_I, k, "fp8"), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    ws_a = torch.empty(max(1, C.sparse_attn_workspace_size(1, T, H, 128, k, W)), dtype=torch.uint8, device=dev)
    ops = [
        ("compress_kv", lambda: st.__setitem__("E", C.csa_compress(c["c_a"], c["c_b"], c["z_a"], c["z_b"], 4))),
        ("compress_index_keys", lambda: st.__setitem__("KI", C.csa_compress(ci["a"], ci["b"], ci["za"], ci["zb"], 4,
                                                                             out_fmt="fp8"))),
        ("indexer_topk", lambda: C.indexer_topk(qi, qs, w, st["KI"][0], st["KI"][1], "fp8", q_pos, 4, k, d_I,
                                                ws=ws_i, idx_out=st["idx"])),
        ("sparse_attn", lambda: C.sparse_attn_fwd(q, st["E"], st["idx"], c["c_a"], win_start, sink, q_pos, W, 1.0,
                                                  ws=ws_a, out=out)),
    ]
    t = time_ops(torch, ops, iters)
    split = {kn: call_kernel_ms(torch, C, ops[2][1], kn) for kn in ("index_score", "topk")}
    bf = bf16_score_variant(torch, C, iters, lambda ws_b: C.indexer_topk(
        qi, qs, w, st["KI"][0], st["KI"][1], "fp8", q_pos, 4, k, d_I, ws=ws_b, idx_out=st["idx"], bf16_scores=True),
        C.indexer_topk_workspace_size(1, T, N, H_I, d_I, k, "fp8", bf16_scores=True))
    p = np.arange(T, dtype=np.int64)
    n = np.minimum(N, (p + 1) // 4)
    keys = np.minimum(k, n) + np.minimum(p + 1, W)
    fl_i, fl_a = index_flops(n, H_I, d_I), attn_flops(keys, H)
    return {"workload": "csa_prefill_bf16_T65536", "tokens": T, "heads": H, "top_k": k, "index": "64x128 fp8",
            "ms": {kk: round(v, 4) for kk, v in t.items()}, "layer_ms": round(sum(t.values()), 4),
            "indexer_tflop": round(fl_i / 1e12, 4), "attn_tflop": round(fl_a / 1e12, 4),
            "indexer_tflop_s": round(fl_i / (t["indexer_topk"] * 1e-3) / 1e12, 2),
            "indexer_split_ms": {kn: (None if v is None else round(v, 4)) for kn, v in split.items()},
            "index_score_tflop_s": (None if not split["index_score"] else
                                    round(fl_i / (split["index_score"] * 1e-3) / 1e12, 2)),
            "sparse_attn_tflop_s": round(fl_a / (t["sparse_attn"] * 1e-3) / 1e12, 2),
            "sparse_attn_frac_bf16_peak": round(fl_a / (t["sparse_attn"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "indexer_bf16_scores": bf}


def decode_append(torch, C, syn, iters):
    """Decode-time cache maintenance of the 1M-context layer pair, B = 8: each
    step appends one token per sequence to the CSA KV cache (bf16 entries), the
    CSA indexer-key cache (fp4 entries + E8M0 scales) and the HCA cache (bf16),
    through their state rings, and each layer's new window row to its window
    ring (128 rows). The positions end a 128-token block, so every call writes
    a CSA entry and an HCA entry (the most work a step can do)."""
    dev, bf = "cuda", torch.bfloat16
    B, L, W = 8, 1 << 20, 128
    N, NH = L // 4, L // 128
    s = 5000
    rows = [syn.normal_device(s + i, (B, W), dev, bf) for i in range(10)]
    pos = torch.full((B,), L - 1, dtype=torch.int32, device=dev)
    E = torch.empty(B, N, W, dtype=bf, device=dev)
    KI = torch.empty(B, N, W // 2, dtype=torch.uint8, device=dev)
    KIs = torch.empty(B, N, W // 32, dtype=torch.uint8, device=dev)
    EH = torch.empty(B, NH, W, dtype=bf, device=dev)
    st_kv = syn.normal_device(s + 20, (B, 8, 4, W), dev, bf)
    st_ix = syn.normal_device(s + 21, (B, 8, 4, W), dev, bf)
    st_h = syn.normal_device(s + 22, (B, 128, 2, W), dev, bf)
    win_csa = syn.normal_device(s + 23, (B, 128, W), dev, bf)
    win_hca = syn.normal_device(s + 24, (B, 128, W), dev, bf)
    ops = [
        ("csa_kv", lambda: C.csa_compress_append(*rows[0:4], pos, st_kv, E, None, 4)),
        ("csa_index_keys_fp4", lambda: C.csa_compress_append(*rows[4:8], pos, st_ix, KI, KIs, 4)),
        ("hca", lambda: C.hca_compress_append(rows[8], rows[9], pos, st_h, EH, 128)),
        ("window_rows", lambda: (C.window_append(rows[0], pos, win_csa), C.window_append(rows[8], pos, win_hca))),
    ]
    # device time per op and per step: 50 steps captured in one graph,
    # replayed (a single call is shorter than its host-side launch path, and a
    # graph replay has a fixed cost of its own)
    per_graph, reps = 50, 10
    def graph_us(fns):
        for f in fns:
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                for f in fns:
                    f()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * per_graph) * 1e3
    t = {name: graph_us([f]) for name, f in ops}
    step = graph_us([f for _, f in ops])
    # bytes a step touches: ring rows read (CSA 7 earlier tokens x 4 streams,
    # HCA 127 tokens x 2 streams), the new rows read and written to the ring,
    # the entries written
    rb = W * 2
    byts = B * (2 * (7 * 4 + 4 + 4) * rb + (127 * 2 + 2 + 2) * rb + rb + W // 2 + W // 32 + rb + 2 * 2 * rb)
    return {"workload": "decode_append_pair_1m_ctx", "batch": B, "context": L,
            "us": {k: round(v, 2) for k, v in t.items()}, "step_us": round(step, 2), "step_bytes": byts,
            "timing": "hip graph replay"}


def prefill_hca(torch, C, syn, iters):
    """Single HCA layer prefill, bf16, T = 131,072: 128:1 compression to 1024
    entries, then dense attention (64 heads) over all visible entries plus the
    128-token window and the sink."""
    dev, bf = "cuda", torch.bfloat16
    T, H, W = 131072, 64, 128
    s = 3000
    cc = syn.normal_device(s, (1, T, 128), dev, bf)
    zz = syn.normal_device(s + 1, (1, T, 128), dev, bf)
    q = syn.normal_device(s + 2, (1, T, H, 128), dev, bf, scale=1 / np.sqrt(128))
    sink = syn.normal_device(s + 3, (H,), dev)
    q_pos = torch.arange(T, dtype=torch.int32, device=dev)[None]
    win_start = torch.zeros(1, dtype=torch.int32, device=dev)
    N = T // 128
    st = {"E": C.hca_compress(cc, zz, 128)}
    out = torch.empty_like(q)
    ws = torch.empty(max(1, C.dense_attn_workspace_size(1, T, N, H, 128, W)), dtype=torch.uint8, device=dev)
    ops = [("compress", lambda: st.__setitem__("E", C.hca_compress(cc, zz, 128))),
           ("dense_attn", lambda: C.dense_compressed_attn_fwd(q, st["E"], cc, win_start, sink, q_pos, 128, W, 1.0,
                                                              ws=ws, out=out))]
    t = time_ops(torch, ops, iters)
    p = np.arange(T, dtype=np.int64)
    keys = np.minimum(N, (p + 1) // 128) + np.minimum(p + 1, W)
    fl = attn_flops(keys, H)
    return {"workload": "hca_prefill_bf16_T131072", "tokens": T, "heads": H,
            "ms": {kk: round(v, 4) for kk, v in t.items()}, "layer_ms": round(sum(t.values()), 4),
            "attn_tflop": round(fl / 1e12, 4), "dense_attn_tflop_s": round(fl / (t["dense_attn"] * 1e-3) / 1e12, 2),
            "dense_attn_frac_bf16_peak": round(fl / (t["dense_attn"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}


def prefill_chunk(torch, C, syn, iters):
    """CSA + HCA layer pair for an 8192-query prefill chunk at the end of a
    1,048,576-token context: indexer over 262,144 fp4 entries (top-1024),
    sparse attention and HCA dense attention over 8192 entries, 128 heads."""
    dev, bf = "cuda", torch.bfloat16
    L, Tq, H, H_I, d_I, k, W = 1 << 20, 8192, 128, 64, 128, 1024, 128
    N, NH = L // 4, L // 128
    s = 4000
    ki32 = syn.normal_device(s, (1, N, d_I), dev)
    kc, ks = C.csa_quantize_rows(ki32, "fp4")
    del ki32
    E = syn.normal_device(s + 1, (1, N, 128), dev, bf)
    xw = syn.normal_device(s + 2, (1, Tq + W - 1, 128), dev, bf)
    q = syn.normal_device(s + 3, (1, Tq, H, 128), dev, bf, scale=1 / np.sqrt(128))
    qi32 = syn.normal_device(s + 4, (1, Tq, H_I, d_I), dev)
    qi, qs = C.csa_quantize_rows(qi32, "fp4")
    del qi32
    w = syn.uniform_device(s + 5, (1, Tq, H_I), dev)
    sink = syn.normal_device(s + 6, (H,), dev)
    Eh = syn.normal_device(s + 7, (1, NH, 128), dev, bf)
    xh = syn.normal_device(s + 8, (1, Tq + W - 1, 128), dev, bf)
    qh = syn.normal_device(s + 9, (1, Tq, H, 128), dev, bf, scale=1 / np.sqrt(128))
    sinkh = syn.normal_device(s + 10, (H,), dev)
    q_pos = torch.arange(L - Tq, L, dtype=torch.int32, device=dev)[None]
    win_start = torch.full((1,), L - Tq - W + 1, dtype=torch.int32, device=dev)
    idx = torch.empty(1, Tq, k, dtype=torch.int32, device=dev)
    ws_i = torch.empty(C.indexer_topk_workspace_size(1, Tq, N, H_I, d_I, k, "fp4"), dtype=torch.uint8, device=dev)
    out, outh = torch.empty_like(q), torch.empty_like(qh)
    ws_a = torch.empty(max(1, C.sparse_attn_workspace_size(1, Tq, H, 128, k, W)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, C.dense_attn_workspace_size(1, Tq, NH, H, 128, W)), dtype=torch.uint8, device=dev)
    ops = [("indexer_topk", lambda: C.indexer_topk(qi, qs, w, kc, ks, "fp4", q_pos, 4, k, d_I, ws=ws_i,
                                                   idx_out=idx)),
           ("sparse_attn", lambda: C.sparse_attn_fwd(q, E, idx, xw, win_start, sink, q_pos, W, 1.0, ws=ws_a,
                                                     out=out)),
           ("dense_attn", lambda: C.dense_compressed_attn_fwd(qh, Eh, xh, win_start, sinkh, q_pos, 128, W, 1.0,
                                                              ws=ws_d, out=outh))]
    t = time_ops(torch, ops, iters)
    split = {kn: call_kernel_ms(torch, C, ops[0][1], kn) for kn in ("index_score", "topk")}
    bf = bf16_score_variant(torch, C, iters, lambda ws_b: C.indexer_topk(
        qi, qs, w, kc, ks, "fp4", q_pos, 4, k, d_I, ws=ws_b, idx_out=idx, bf16_scores=True),
        C.indexer_topk_workspace_size(1, Tq, N, H_I, d_I, k, "fp4", bf16_scores=True))
    p = np.arange(L - Tq, L, dtype=np.int64)
    n = np.minimum(N, (p + 1) // 4)
    nh = np.minimum(NH, (p + 1) // 128)
    fl_i = index_flops(n, H_I, d_I)
    fl_a = attn_flops(np.minimum(k, n) + W, H)
    fl_d = attn_flops(nh + W, H)
    return {"workload": "csa_hca_prefill_chunk_8192q_1m_ctx", "queries": Tq, "context": L, "heads": H,
            "ms": {kk: round(v, 4) for kk, v in t.items()}, "pair_ms": round(sum(t.values()), 4),
            "indexer_tflop": round(fl_i / 1e12, 3), "indexer_tflop_s": round(fl_i / (t["indexer_topk"] * 1e-3) / 1e12, 2),
            "indexer_split_ms": {kn: (None if v is None else round(v, 4)) for kn, v in split.items()},
            "index_score_tflop_s": (None if not split["index_score"] else
                                    round(fl_i / (split["index_score"] * 1e-3) / 1e12, 2)),
            "sparse_attn_tflop_s": round(fl_a / (t["sparse_attn"] * 1e-3) / 1e12, 2),
            "dense_attn_tflop_s": round(fl_d / (t["dense_attn"] * 1e-3) / 1e12, 2),
            "dense_attn_frac_bf16_peak": round(fl_d / (t["dense_attn"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "indexer_bf16_scores": bf}


def attn_bwd_flops(n_keys, H, d=128):
    """S, dP, dQ and the two key-row products: 10 flops per (query, key, head, channel)."""
    return float(np.sum(n_keys, dtype=np.float64)) * H * d * 10


def bwd_csa(torch, C, syn, iters):
    """CSA core-attention backward, T = 65,536, 64 heads, top-512 selected by the
    fp8 indexer plus the 128-token window and the sink (the prefill layer's
    shapes); the forward's output and log-sum-exp are computed once in setup."""
    dev, bf = "cuda", torch.bfloat16
    T, H, H_I, d_I, k, W = 65536, 64, 64, 128, 512, 128
    s = 6000
    c = {n: syn.normal_device(s + i, (1, T, 128), dev, bf) for i, n in enumerate(["c_a", "c_b", "z_a", "z_b"])}
    ci = {n: syn.normal_device(s + 10 + i, (1, T, d_I), dev, bf) for i, n in enumerate(["a", "b", "za", "zb"])}
    q = syn.normal_device(s + 20, (1, T, H, 128), dev, bf, scale=1 / np.sqrt(128))
    qi32 = syn.normal_device(s + 21, (1, T, H_I, d_I), dev)
    qi, qs = C.csa_quantize_rows(qi32, "fp8")
    del qi32
    w = syn.uniform_device(s + 22, (1, T, H_I), dev)
    sink = syn.normal_device(s + 23, (H,), dev)
    dout = syn.normal_device(s + 24, (1, T, H, 128), dev, bf)
    q_pos = torch.arange(T, dtype=torch.int32, device=dev)[None]
    win_start = torch.zeros(1, dtype=torch.int32, device=dev)
    E = C.csa_compress(c["c_a"], c["c_b"], c["z_a"], c["z_b"], 4)
    KI = C.csa_compress(ci["a"], ci["b"], ci["za"], ci["zb"], 4, out_fmt="fp8")
    idx = C.indexer_topk(qi, qs, w, KI[0], KI[1], "fp8", q_pos, 4, k, d_I)
    out, lse = C.sparse_attn_fwd(q, E, idx, c["c_a"], win_start, sink, q_pos, W, 1.0, want_lse=True)
    N = T // 4
    ws = torch.empty(C.sparse_attn_bwd_workspace_size(1, T, N, T, H, 128, k, W), dtype=torch.uint8, device=dev)
    fn = lambda: C.sparse_attn_bwd(q, E, idx, c["c_a"], win_start, sink, q_pos, out, lse, dout, W, 1.0, ws=ws)
    t = time_ops(torch, [("sparse_attn_bwd", fn)], iters)["sparse_attn_bwd"]
    main = call_kernel_ms(torch, C, fn, "attn_bwd")
    p = np.arange(T, dtype=np.int64)
    keys = np.minimum(k, np.minimum(N, (p + 1) // 4)) + np.minimum(p + 1, W)
    fl = attn_bwd_flops(keys, H)
    return {"workload": "csa_attn_bwd_bf16_T65536", "tokens": T, "heads": H, "top_k": k, "ms": round(t, 4),
            "main_kernel_ms": None if main is None else round(main, 4), "tflop": round(fl / 1e12, 4),
            "tflop_s": round(fl / (t * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(fl / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "main_kernel_tflop_s": None if not main else round(fl / (main * 1e-3) / 1e12, 2),
            "workspace_gb": round(ws.numel() / 1e9, 2)}


def bwd_hca(torch, C, syn, iters):
    """HCA core-attention backward, T = 131,072, 64 heads, every visible entry
    of 1024 plus the window and the sink."""
    dev, bf = "cuda", torch.bfloat16
    T, H, ratio, W = 131072, 64, 128, 128
    N = T // ratio
    s = 7000
    q = syn.normal_device(s, (1, T, H, 128), dev, bf, scale=1 / np.sqrt(128))
    E = syn.normal_device(s + 1, (1, N, 128), dev, bf)
    xw = syn.normal_device(s + 2, (1, T, 128), dev, bf)
    sink = syn.normal_device(s + 3, (H,), dev)
    dout = syn.normal_device(s + 4, (1, T, H, 128), dev, bf)
    q_pos = torch.arange(T, dtype=torch.int32, device=dev)[None]
    win_start = torch.zeros(1, dtype=torch.int32, device=dev)
    out, lse = C.dense_compressed_attn_fwd(q, E, xw, win_start, sink, q_pos, ratio, W, 1.0, want_lse=True)
    ws = torch.empty(C.dense_attn_bwd_workspace_size(1, T, N, T, H, 128, W), dtype=torch.uint8, device=dev)
    fn = lambda: C.dense_compressed_attn_bwd(q, E, xw, win_start, sink, q_pos, out, lse, dout, ratio, W, 1.0, ws=ws)
    t = time_ops(torch, [("dense_attn_bwd", fn)], iters)["dense_attn_bwd"]
    main = call_kernel_ms(torch, C, fn, "attn_bwd")
    p = np.arange(T, dtype=np.int64)
    keys = np.minimum(N, (p + 1) // ratio) + np.minimum(p + 1, W)
    fl = attn_bwd_flops(keys, H)
    return {"workload": "hca_attn_bwd_bf16_T131072", "tokens": T, "heads": H, "ms": round(t, 4),
            "main_kernel_ms": None if main is None else round(main, 4), "tflop": round(fl / 1e12, 4),
            "tflop_s": round(fl / (t * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(fl / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "main_kernel_tflop_s": None if not main else round(fl / (main * 1e-3) / 1e12, 2),
            "workspace_gb": round(ws.numel() / 1e9, 2)}


def proj(torch, C, syn, iters):
    """Projections around the attention core for one 8,192-token prefill
    chunk, bf16 MFMA GEMMs: the grouped output projection (128 heads x 128 in
    8 groups, rank 1024 per group, model width 7168), the shared-latent
    query projections (7168 -> 1536 latent -> 128 x 128 attention queries and
    64 x 128 indexer queries) and the compressor's input streams (KV and gate
    streams of the KV and index-key compressors, 8 x 128, from 7168). The sizes are a reading: the pages give the
    structure, not these widths."""
    dev, bf = "cuda", torch.bfloat16
    T, H, d, G, r, D, r_q, H_I = 8192, 128, 128, 8, 1024, 7168, 1536, 64
    s = 8000
    o = syn.normal_device(s, (T, H, d), dev, bf)
    wg = syn.normal_device(s + 1, (G, r, H // G * d), dev, bf, scale=1 / np.sqrt(H // G * d))
    wo = syn.normal_device(s + 2, (D, G * r), dev, bf, scale=1 / np.sqrt(G * r))
    x = syn.normal_device(s + 3, (T, D), dev, bf)
    wdq = syn.normal_device(s + 4, (r_q, D), dev, bf, scale=1 / np.sqrt(D))
    wuq = syn.normal_device(s + 5, (H * d, r_q), dev, bf, scale=1 / np.sqrt(r_q))
    wiq = syn.normal_device(s + 6, (H_I * d, r_q), dev, bf, scale=1 / np.sqrt(r_q))
    out = torch.empty(T, D, dtype=bf, device=dev)
    ws_o = torch.empty(C.grouped_out_proj_workspace_size(T, G, r), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(C.query_proj_shared_workspace_size(T, r_q), dtype=torch.uint8, device=dev)
    # the compressor's KV and gate streams and the indexer's key streams: 8 x 128
    wkv = syn.normal_device(s + 7, (8, d, D), dev, bf, scale=1 / np.sqrt(D))
    streams = torch.empty(8, T, d, dtype=bf, device=dev)
    ops = [("grouped_out_proj", lambda: C.grouped_out_proj(o, wg, wo, out=out, ws=ws_o)),
           ("query_proj_shared", lambda: C.query_proj_shared(x, wdq, wuq, wiq, ws=ws_q)),
           ("kv_proj", lambda: C.kv_proj(x, wkv, out=streams))]
    t = time_ops(torch, ops, iters)
    fl_o = 2.0 * T * H * d * r + 2.0 * T * G * r * D
    fl_q = 2.0 * T * D * r_q + 2.0 * T * r_q * (H + H_I) * d
    fl_kv = 2.0 * T * D * 8 * d
    res = {"workload": "projections_bf16_T8192", "tokens": T, "ms": {k: round(v, 4) for k, v in t.items()},
           "grouped_out_proj": {"heads": H, "groups": G, "rank": r, "width": D, "tflop": round(fl_o / 1e12, 4),
                                "tflop_s": round(fl_o / (t["grouped_out_proj"] * 1e-3) / 1e12, 1),
                                "frac_bf16_peak": round(fl_o / (t["grouped_out_proj"] * 1e-3) / 1e12
                                                        / BF16_PEAK_TFLOPS, 4)},
           "query_proj_shared": {"latent": r_q, "tflop": round(fl_q / 1e12, 4),
                                 "tflop_s": round(fl_q / (t["query_proj_shared"] * 1e-3) / 1e12, 1),
                                 "frac_bf16_peak": round(fl_q / (t["query_proj_shared"] * 1e-3) / 1e12
                                                         / BF16_PEAK_TFLOPS, 4)},
           "kv_proj": {"streams": 8, "width": d, "tflop": round(fl_kv / 1e12, 4),
                       "tflop_s": round(fl_kv / (t["kv_proj"] * 1e-3) / 1e12, 1),
                       "frac_bf16_peak": round(fl_kv / (t["kv_proj"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
    return res


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="rotated cache copies (defeats the Infinity Cache)")
    ap.add_argument("--extras", default="decode_batches,decode4,decode_bf16,decode_append,prefill_csa,prefill_hca,"
                                        "prefill_chunk,bwd_csa,bwd_hca,"
                                        "proj",
                    help="comma list of decode_batches,decode4,decode_bf16,decode_append,prefill_csa,prefill_hca,"
                         "prefill_chunk,bwd_csa,bwd_hca,proj or 'none'")
    ap.add_argument("--prefill-iters", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed region, copy 512 MiB device to device once (the reference "
                         "transfer for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the sharded path exists only as "
              "a design. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import csa_synth as syn
    import long_context_attention_csa_amd as C
    from oracle import csa_oracle as O   # CPU-baseline leg only

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    st, ms, wall, kt = run_decode(torch, C, syn, O, args, "pair1m")
    B = st["B"]
    qps = B / (ms * 1e-3)
    dom_us = st["score_us"]
    # a score-stage launch reads the keys, queries and weights and writes one
    # float32 score per (sequence, entry)
    dom_bytes = st["bytes_index_score"] + B * st["N"] * 4
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    step_gbs = st["bytes"] / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp4",
        "data": "synthetic",
        "config": {"workload": st["name"], "batch": B, "context": st["L"], "csa_entries": st["N"],
                   "hca_entries": st["NH"], "heads": st["H"], "head_dim": 128, "index_heads": st["H_I"],
                   "index_dim": st["d_I"], "index_keys": "fp4 e2m1 + E8M0 per 32", "top_k": st["k"],
                   "window": 128, "kv": "bf16", "cache_copies": args.copies,
                   "timing": "eager" if args.eager else "hip graph replay"},
        "hbm_tb_s": round(st["bytes"] / (ms * 1e-3) / 1e12, 3),
        "step_bytes": st["bytes"],
        "wall_ms_per_step": round(wall, 5),
        "kernel_us": {k_: (None if v is None else round(v * 1e3, 2)) for k_, v in kt.items()},
        "kernel_us_note": "per-launch HIP events around each kernel of eager steps (include the launch itself)",
        "roofline": {"bound": "hbm", "kernel": "k_index_score_dec (fp4 keys; score-stage launches)",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("k_index_score",
                                                 "long_context_attention_csa_amd/csrc/indexer.hip"),
                     "bytes_per_launch": dom_bytes, "us_per_launch": round(dom_us, 2),
                     "timing": "48 back-to-back score-stage launches over the rotated cache copies in one HIP "
                               "graph, HIP events on its stream"},
        "step_roofline": {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(step_gbs / HBM_PEAK_GBS, 4), "bytes_per_step": st["bytes"]},
        "index_recall_vs_float32": {"format": st["fmt"], "rows": st["recall"],
                                    "note": "selection on quantised operands vs on the same operands in float32"},
        "pages_claims": PAGES_CLAIMS,
    }
    if not args.no_cpu_baseline:
        done, spent = cpu_baseline_decode(O, st, args.cpu_seconds)
        result["cpu_baseline"] = {"value": round(done / spent, 3), "unit": "queries/s",
                                  "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                                  "sample": f"{done} single-sequence decode steps of the whole CSA+HCA pair "
                                            f"(float64 NumPy, 2 sequences of the batch cycled), {spent:.1f} s"}
    extras = {}
    wanted = [] if args.extras == "none" else [x for x in args.extras.split(",") if x]
    del st
    torch.cuda.empty_cache()
    if "decode_bf16" in wanted:
        # the same decode pair with bfloat16 index scores (indexer_topk_bf16_scores)
        stb, msb, wallb, ktb = run_decode(torch, C, syn, O, args, "pair1m_bf16")
        extras["csa_hca_decode_pair_1m_ctx_bf16_scores"] = {
            "queries_per_s": round(stb["B"] / (msb * 1e-3), 1), "ms_per_step": round(msb, 5),
            "kernel_us": {k_: (None if v is None else round(v * 1e3, 2)) for k_, v in ktb.items()}}
        del stb
        torch.cuda.empty_cache()
    if "decode_batches" in wanted:
        r = decode_batches(torch, C, syn, args.steps, args.warmup)
        extras[r["workload"]] = r
    if "decode4" in wanted:
        st4, ms4, wall4, kt4 = run_decode(torch, C, syn, O, args, "decode4")
        extras["csa_decode_262k_ctx"] = {
            "batch": st4["B"], "queries_per_s": round(st4["B"] / (ms4 * 1e-3), 1), "ms_per_step": round(ms4, 5),
            "hbm_tb_s": round(st4["bytes"] / (ms4 * 1e-3) / 1e12, 3),
            "index_score_gb_s": round((st4["bytes_index_score"] + st4["B"] * st4["N"] * 4) / (st4["score_us"] * 1e-6)
                                      / 1e9, 1),
            "index_score_us": round(st4["score_us"], 2),
            "index_recall_vs_float32": {"format": st4["fmt"], "rows": st4["recall"]},
            "kernel_us": {k_: (None if v is None else round(v * 1e3, 2)) for k_, v in kt4.items()}}
        del st4
        torch.cuda.empty_cache()
    for key, fn in (("decode_append", decode_append), ("prefill_csa", prefill_csa), ("prefill_hca", prefill_hca),
                    ("prefill_chunk", prefill_chunk), ("bwd_csa", bwd_csa), ("bwd_hca", bwd_hca), ("proj", proj)):
        if key in wanted:
            r = fn(torch, C, syn, args.prefill_iters)
            log(f"[bench] {r['workload']}: {r}")
            extras[r["workload"]] = r
            torch.cuda.empty_cache()
    if extras:
        result["extras"] = extras
    if args.calib_copy:
        a = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        bcopy = torch.empty_like(a)
        torch.cuda.synchronize()
        bcopy.copy_(a)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = 512 << 20
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
