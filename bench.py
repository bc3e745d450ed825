"""Benchmark: load-balanced split-KV decode attention on one MI355X.

A step is one decode step of the whole path over one batch: hpcattn_plan
once, then hpcattn_decode + hpcattn_combine for every layer, each layer with
its own KV pool (so the 256 MB Infinity Cache cannot serve repeats).  Inputs
are resident in HBM before the timed region starts.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--num-bins P]
                    [--min-tiles m] [--ablation] [--no-cpu-baseline] [--no-extras]

NAME: mixed (default), single_long, heavy_tail, heavy_tail_long_first,
heavy_tail_long_last, fp8, mtp, mtp_fp8, mixed_shard, or prologue.

Prints one JSON line.  `value` is the step's KV-read throughput (live KV
bytes of all layers / step time), the step replayed from a HIP graph as a
serving loop would (--eager launches each kernel from the host instead);
`roofline` is for the decode kernel, its average launch time taken with HIP
events around a graph of back-to-back decode launches on the stream they run
on; `cpu_baseline` is the fp64 oracle on the host cores over a bounded sample
of the same workload.  The default (mixed) run then adds `heavy_tail`: the
heavy-tail batch in its three orders, dynamic decode + combine (two launches
and fused) against every point of the static split-KV sweep; and
`mixed_shard`: the step at one GPU's head shard of the mixed batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step + KV-read GB/s (% HBM peak), mixed-length GQA batch"
HBM_PEAK_GBS = 8000.0
WARM_GPU_MS = 100.0         # least GPU time of untimed graph replays before timed steps
FIRST_WARM_GPU_MS = 2000.0  # ... before a process's first timed steps
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SRC = os.path.join(ROOT, "load_balanced_split_amd", "csrc", "decode.hip")

DESCRIPTIONS = {
    "mixed": "mixed-length: 64 requests, KV lens log-uniform in [256, 32768] (seed 0), "
             "8 KV / 64 Q heads, head_dim 128, bf16, page 64, shuffled pages, "
             "32 layers with distinct KV pools, one task map per step",
    "single_long": "single long: 1 request of 131072 tokens, 8 KV / 64 Q heads, head_dim 128, "
                   "bf16, page 64, shuffled pages, 4 rotating KV pools",
    "heavy_tail": "heavy-tail: 120 requests of 1024+-10% and 8 of 65536 tokens, 8 KV / 64 Q "
                  "heads, head_dim 128, bf16, page 64, 4 rotating KV pools",
    "heavy_tail_long_first": "heavy-tail, long requests first: the heavy-tail lengths with "
                             "the 8 requests of 65536 tokens at batch positions 0-7, 8 KV / "
                             "64 Q heads, head_dim 128, bf16, page 64, 4 rotating KV pools",
    "heavy_tail_long_last": "heavy-tail, long requests last: the heavy-tail lengths with the 8 "
                            "requests of 65536 tokens at batch positions 120-127, 8 KV / 64 Q "
                            "heads, head_dim 128, bf16, page 64, 4 rotating KV pools",
    "mixed_shard": "mixed-length head shard (one GPU of 8-way head parallelism): 64 requests, "
                   "KV lens log-uniform in [256, 32768] (seed 0), 1 KV / 8 Q heads, head_dim "
                   "128, bf16, page 64, 32 layers with distinct KV pools, one task map per step",
    "fp8": "fp8 KV: 32 requests, KV lens log-uniform in [1024, 131072], 8 KV / 64 Q heads, "
           "head_dim 128, e4m3 Q/K/V with per-token per-head fp32 scales, page 64, "
           "4 rotating KV pools",
    "mtp": "draft verify: the mixed-length batch (64 requests, KV lens log-uniform in "
           "[256, 32768], seed 0) with 6 query rows per request (1 + 5 drafts, causal among "
           "themselves), 8 KV / 64 Q heads, head_dim 128, bf16, page 64, 32 layers with "
           "distinct KV pools, one task map per step",
    "mtp_fp8": "draft verify, fp8 KV: the fp8 batch (32 requests, KV lens log-uniform in "
               "[1024, 131072]) with 6 query rows per request (1 + 5 drafts), 8 KV / 64 Q "
               "heads, head_dim 128, e4m3 Q/K/V with per-token per-head fp32 scales, page 64, "
               "4 rotating KV pools",
}


def note(*a):
    """A progress line on stderr (the JSON result alone goes to stdout)."""
    print("#", *a, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed", choices=sorted(DESCRIPTIONS) + ["prologue"])
    ap.add_argument("--num-bins", type=int, default=None)
    ap.add_argument("--min-tiles", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None,
                    help="layers (distinct KV pools) per step; default 32 for mixed, else 1")
    ap.add_argument("--pools", type=int, default=4,
                    help="rotating KV pools for the one-layer workloads")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--ablation", action="store_true",
                    help="also sweep the static split-KV baseline on the same inputs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="with the mixed workload: skip the heavy-tail order sweep and the "
                         "head-shard step that follow the headline")
    ap.add_argument("--warm-ms", type=float, default=FIRST_WARM_GPU_MS,
                    help="least GPU time (ms) of untimed step replays before the first timed "
                         "region; later regions get min(this, %g) (0 under rocprofv3 --pmc, "
                         "which serialises every dispatch)" % WARM_GPU_MS)
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from the host instead of replaying the step "
                         "from a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--oracle-layer", action="store_true",
                    help="instead of the benchmark: time the fp64 CPU oracle on one full layer "
                         "of the workload (all host cores, then 1 thread; median of 3 each), "
                         "print one JSON line; needs no GPU")
    ap.add_argument("--calibrate", action="store_true",
                    help="instead of the benchmark: time a plain 1 GiB device copy and a "
                         "4 GiB read-reduce (HBM read probe), print one JSON line")
    return ap.parse_args()


def calibrate():
    """Reference kernels of known traffic: torch's device copy of 1 GiB (the
    scale for the HBM byte counters) and a 4 GiB read-reduce (the achievable
    read bandwidth)."""
    import torch
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    n_copy = 1 << 30
    x = torch.zeros(n_copy // 2, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    big = torch.zeros((1 << 32) // 2, dtype=torch.bfloat16, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(reps):
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return statistics.median(ts)

    from load_balanced_split_amd import hpcattn as H
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    copy_ms = timed(lambda: y.copy_(x), 5)
    read_ms = timed(lambda: big.sum(dtype=torch.float32), 5)
    probe = {}
    for nt in (False, True):
        for wg in (512, 1024, 2048, 4096, 8192, 16384, 32768):
            ms = timed(lambda: H.hpcattn_probe_stream_read(big, wg, sink, nt), 5)
            probe["%s%d" % ("nt" if nt else "plain", wg)] = round(big.numel() * 2 / ms / 1e6, 1)
    chunked = {}
    for wg in (512, 768, 1024, 1536, 2048, 4096, 8192, 16384):
        ms = timed(lambda: H.hpcattn_probe_stream_read(big, wg, sink, True, True), 5)
        chunked["nt_chunk16k_%d" % wg] = round(big.numel() * 2 / ms / 1e6, 1)
    best = max(probe, key=probe.get)
    print(json.dumps({
        "calibration": "device copy of %d bytes; read-reduce and stream-read probe of %d bytes"
                       % (n_copy, big.numel() * 2),
        "copy_bytes": n_copy, "copy_ms": round(copy_ms, 4),
        "copy_GBs_read_plus_write": round(2 * n_copy / copy_ms / 1e6, 1),
        "read_bytes": big.numel() * 2, "torch_sum_GBs": round(big.numel() * 2 / read_ms / 1e6, 1),
        "stream_read_GBs_by_loads_workgroups": probe, "stream_read_best_GBs": probe[best],
        "stream_read_best": best, "chunked_16k_read_GBs_by_workgroups": chunked,
        "chunked_16k_read_best_GBs": max(chunked.values())}), flush=True)


def oracle_layer(name: str, seed: int, runs: int = 3):
    """The fp64 oracle, as it stands, on one whole layer of a workload: every
    (request, KV head) pair, on all host cores and then on one thread, the
    median of `runs` passes each.  Inputs are built on the host."""
    import numpy as np

    import oracle
    from load_balanced_split_amd import workloads as wl

    prob = wl.make_problem(name, seed=seed, device="cpu", layers=1)
    w = prob.workload
    h = dict(q=wl.as_numpy(prob.q), k_pages=wl.as_numpy(prob.k_pages[0]),
             v_pages=wl.as_numpy(prob.v_pages[0]))
    if w.kv_dtype == "fp8":
        h.update(q_scale=wl.as_numpy(prob.q_scale), k_scale=wl.as_numpy(prob.k_scale[0]),
                 v_scale=wl.as_numpy(prob.v_scale[0]))
    kv = int(np.asarray(prob.seq_lens).sum()) * wl.kv_bytes_per_token(w)

    def layer():
        t0 = time.perf_counter()
        oracle.attention(h["q"], h["k_pages"], h["v_pages"], prob.page_table, prob.seq_lens,
                         num_kv_heads=w.num_kv_heads, sm_scale=prob.sm_scale,
                         q_scale=h.get("q_scale"), k_scale=h.get("k_scale"),
                         v_scale=h.get("v_scale"))
        dt = time.perf_counter() - t0
        note("oracle layer pass: %.2f s" % dt)
        return dt

    cores = oracle.max_threads()
    note("oracle layer", name, "on", cores, "threads")
    t_all = statistics.median(layer() for _ in range(runs))
    oracle.set_threads(1)
    try:
        note("oracle layer", name, "on 1 thread")
        t_one = statistics.median(layer() for _ in range(runs))
    finally:
        oracle.set_threads(cores)
    print(json.dumps({"oracle_layer": DESCRIPTIONS.get(name, name), "workload": name,
                      "kv_bytes": kv, "runs": runs, "cores": cores,
                      "us_all_cores": round(t_all * 1e6), "gbs_all_cores": round(kv / t_all / 1e9, 3),
                      "us_one_thread": round(t_one * 1e6), "gbs_one_thread": round(kv / t_one / 1e9, 3),
                      "host": _cpu_model()}), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def prologue_bench(reps=20):
    """The fused prologue (QK-Norm, RoPE, Hadamard, quantisation, KV store)
    at a decode shape (64 tokens, one per request) and a prefill shape
    (16384 tokens), 64 Q / 8 KV heads, D = 128, bf16 in; fp8 and bf16 out.
    Bytes = bf16 QKV read + norm weights + positions / slots + Q, K, V (and
    scales) written; timed as a HIP graph of `reps` launches."""
    import numpy as np
    import torch

    from load_balanced_split_amd import hpcattn as H
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    Hq, Hkv, D = 64, 8, 128
    res = {}
    for T in (64, 16384):
        for fp8 in (True, False):
            num_pages = (T + 63) // 64 + 1
            gen = torch.Generator(device="cuda")
            gen.manual_seed(T)
            qkv = torch.randn((T, (Hq + 2 * Hkv) * D), generator=gen, device="cuda").to(
                torch.bfloat16)
            pos = torch.arange(T, dtype=torch.int32, device="cuda")
            slots = torch.randperm(num_pages * 64, generator=torch.Generator().manual_seed(T))[
                :T].to(torch.int32).cuda()
            w = torch.ones(D, device="cuda")
            dt = torch.uint8 if fp8 else torch.bfloat16
            q_out = torch.empty((T, Hq, D), dtype=dt, device="cuda")
            kp = torch.zeros((num_pages, Hkv, 64, D), dtype=dt, device="cuda")
            vp = torch.zeros_like(kp)
            sc = {}
            if fp8:
                sc = dict(q_scale=torch.empty((T, Hq), device="cuda"),
                          k_scale=torch.zeros((num_pages, Hkv, 64), device="cuda"),
                          v_scale=torch.zeros((num_pages, Hkv, 64), device="cuda"))
            dims = H.hpcattn_prologue_dims(T, Hq, Hkv, D, num_pages,
                                           H.KV_FP8_E4M3 if fp8 else H.KV_BF16,
                                           H.PROLOGUE_ROPE | H.PROLOGUE_HADAMARD, 1e-6, 10000.0)

            def call():
                H.hpcattn_prologue(dims, qkv, pos, slots, q_out, kp, vp, q_norm_w=w,
                                   k_norm_w=w, **sc)
            call()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    call()
            g.replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            b.synchronize()
            us = a.elapsed_time(b) / reps * 1e3
            unfused_us = unfused_prologue_us(qkv, pos, slots, w, kp, vp, sc, Hq, Hkv, D, fp8,
                                             stream, reps)
            esz = 1 if fp8 else 2
            nbytes = (T * (Hq + 2 * Hkv) * D * 2 + 2 * D * 4 + 2 * T * 4
                      + T * (Hq + 2 * Hkv) * D * esz + (T * (Hq + 2 * Hkv) * 4 if fp8 else 0))
            res["T=%d %s" % (T, "fp8" if fp8 else "bf16")] = {
                "us": round(us, 2), "unfused_torch_us": round(unfused_us, 2),
                "speedup_vs_unfused": round(unfused_us / us, 2), "bytes": nbytes,
                "GBs": round(nbytes / us / 1e3, 1),
                "pct_hbm_peak": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1)}
    print(json.dumps({"prologue": "QK-Norm + RoPE + Hadamard + quantise + KV store, "
                                  "64 Q / 8 KV heads, D 128, bf16 in", "results": res}),
          flush=True)


def unfused_prologue_us(qkv, pos, slots, w, kp, vp, sc, Hq, Hkv, D, fp8, stream, reps):
    """The same prologue as separate PyTorch GPU operations (each step a kernel
    with its own HBM round trip), the unfused chain the fused kernel replaces:
    RMSNorm, RoPE from precomputed cos/sin tables, Hadamard as a matmul,
    per-row quantisation, KV scatter.  Timed the same way (HIP graph)."""
    import math

    import scipy.linalg
    import torch
    T = qkv.shape[0]
    half = D // 2
    inv = 10000.0 ** (-2.0 * torch.arange(half, dtype=torch.float64, device="cuda") / D)
    ang = pos.double()[:, None] * inv[None, :]
    cos, sin = ang.cos().float(), ang.sin().float()
    Hd = torch.from_numpy(scipy.linalg.hadamard(D) / math.sqrt(D)).float().cuda()
    q_out = torch.empty((T, Hq, D), dtype=torch.uint8 if fp8 else torch.bfloat16,
                        device="cuda")
    kflat = kp.view(-1, Hkv, D)
    vflat = vp.view(-1, Hkv, D)
    sl = slots.long()

    def step():
        x = qkv.view(T, Hq + 2 * Hkv, D).float()
        q, k, v = x[:, :Hq], x[:, Hq:Hq + Hkv], x[:, Hq + Hkv:]
        q = q * torch.rsqrt(q.pow(2).mean(-1, keepdim=True) + 1e-6) * w
        k = k * torch.rsqrt(k.pow(2).mean(-1, keepdim=True) + 1e-6) * w
        c, s_ = cos[:, None, :], sin[:, None, :]
        q = torch.cat([q[..., :half] * c - q[..., half:] * s_,
                       q[..., half:] * c + q[..., :half] * s_], -1)
        k = torch.cat([k[..., :half] * c - k[..., half:] * s_,
                       k[..., half:] * c + k[..., :half] * s_], -1)
        q = q @ Hd.T
        k = k @ Hd.T
        if fp8:
            outs = []
            for t_ in (q, k, v):
                amax = t_.abs().amax(-1, keepdim=True)
                scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
                outs.append(((t_ / scale).clamp(-448, 448).to(torch.float8_e4m3fn)
                             .view(torch.uint8), scale.squeeze(-1)))
            q_out.copy_(outs[0][0])
            sc["q_scale"].copy_(outs[0][1])
            kflat[sl] = outs[1][0]
            vflat[sl] = outs[2][0]
            sc["k_scale"].view(-1, Hkv)[sl] = outs[1][1]
            sc["v_scale"].view(-1, Hkv)[sl] = outs[2][1]
        else:
            q_out.copy_(q.to(torch.bfloat16))
            kflat[sl] = k.to(torch.bfloat16)
            vflat[sl] = v.to(torch.bfloat16)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            step()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g.replay()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / reps * 1e3


def decode_code_sha256() -> str:
    """sha256 of the decode kernels' source with its // comments and blank
    lines removed: the code a counter summary measured, which an edit of a
    comment does not change."""
    lines = []
    with open(DECODE_SRC, encoding="utf-8") as f:
        for line in f:
            code = line.split("//", 1)[0].rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def traffic_from_profile(workload: str):
    """HBM bytes per decode launch from the committed counter summary of this
    workload, if there is one and it was taken on the current decode code."""
    path = os.path.join(PROFILES, "decode_%s_traffic.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"decode_code_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t:
        return None
    return float(t.group(1)) if decode_code_sha256() == m.group(1) else None


def cpu_baseline(prob, budget_s: float):
    """The fp64 oracle, as it stands, on all host cores over a bounded sample
    of layer 0: whole (request, KV head) pairs in a seeded order, cycling
    over the layer, until the time budget is spent; then the same on one
    thread for a third of the budget.  Returns the KV GB/s they sustained."""
    import numpy as np

    import oracle
    from load_balanced_split_amd import workloads as wl

    w = prob.workload
    h = dict(q=wl.as_numpy(prob.q), k_pages=wl.as_numpy(prob.k_pages[0]),
             v_pages=wl.as_numpy(prob.v_pages[0]), page_table=prob.page_table,
             seq_lens=prob.seq_lens)
    if w.kv_dtype == "fp8":
        h.update(q_scale=wl.as_numpy(prob.q_scale), k_scale=wl.as_numpy(prob.k_scale[0]),
                 v_scale=wl.as_numpy(prob.v_scale[0]))
    rng = np.random.default_rng(7)
    pairs = [(int(b), hh) for b in rng.permutation(len(prob.seq_lens))
             for hh in range(w.num_kv_heads)]
    per_tok_head = wl.kv_bytes_per_token(w) // w.num_kv_heads

    def sample(budget, chunk):
        done_tok, spent, i = 0, 0.0, 0
        while spent < budget:
            sel = [pairs[(i + k) % len(pairs)] for k in range(chunk)]
            t0 = time.perf_counter()
            oracle.attention(h["q"], h["k_pages"], h["v_pages"], h["page_table"],
                             h["seq_lens"], num_kv_heads=w.num_kv_heads,
                             sm_scale=prob.sm_scale, q_scale=h.get("q_scale"),
                             k_scale=h.get("k_scale"), v_scale=h.get("v_scale"), pairs=sel)
            spent += time.perf_counter() - t0
            done_tok += sum(int(prob.seq_lens[b]) for b, _ in sel)
            i += len(sel)
        return done_tok * per_tok_head / spent / 1e9, i, done_tok, spent

    cores = oracle.max_threads()
    gbs, n, tok, spent = sample(budget_s, max(cores, 8))
    oracle.set_threads(1)
    try:
        gbs1, n1, tok1, spent1 = sample(budget_s / 3, 1)
    finally:
        oracle.set_threads(cores)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "layer 0 of the same workload, %d (request, KV head) attention tasks "
                      "(%.2f passes over the layer's %d pairs, %d KV tokens), %.1f s of fp64 "
                      "C/OpenMP work" % (n, n / len(pairs), len(pairs), tok, spent),
            "single_thread": {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1,
                              "sample": "%d attention tasks, %d KV tokens, %.1f s"
                                        % (n1, tok1, spent1)}}


class Clock:
    """HIP-event timing on one stream: graph capture, warm averages of
    back-to-back launches, and the timed region of K steps.

    Warm-up: a GPU left idle by a capture needs some milliseconds to return
    to its running speed (about 25 ms of work on the draft-verify fp8
    workload, whose first 20 steps ran 15% slower than the next ones), and a
    process's first second or so of GPU work can run slower still (the mixed
    step measured 8730 us after 100 ms of warm-up in a process started right
    after another, 8380 us after 2 s).  So the first timed region of the
    process follows untimed replays of at least `first_warm_ms` of GPU time,
    later ones at least min(WARM_GPU_MS, first_warm_ms)."""

    def __init__(self, stream, first_warm_ms, eager=False):
        self.stream = stream
        self.warm_later = min(WARM_GPU_MS, first_warm_ms)
        self.next_warm = first_warm_ms
        self.eager = eager

    def events(self):
        import torch
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def capture(self, fn):
        """Capture fn's launches into a HIP graph on torch's capture stream."""
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def graph_avg_ms(self, fn, count, reps=5, warm=0.0):
        """Average GPU time of one of the `count` launches fn() enqueues, from
        HIP events around replays of a graph holding them back to back,
        after untimed replays for at least `warm` ms of GPU time.  The decode
        graphs are warmed (the capture leaves the GPU idle, as for the step);
        the short combine and plan launches are not: 100 ms of them alone
        measured the combine at twice its time inside the step, so they are
        timed right after a warm decode graph instead."""
        import torch
        g = self.capture(fn)
        a, b = self.events()
        a.record(self.stream)
        g.replay()
        b.record(self.stream)
        b.synchronize()
        for _ in range(math.ceil(warm / max(a.elapsed_time(b), 1e-3))):
            g.replay()
        torch.cuda.synchronize()
        a.record(self.stream)
        for _ in range(reps):
            g.replay()
        b.record(self.stream)
        b.synchronize()
        return a.elapsed_time(b) / (reps * count)

    def timed(self, one_step, steps, warmup, per_graph):
        """Exactly `steps` steps enqueued back to back with no host
        synchronisation between them (as a serving loop enqueues its steps),
        bracketed by a synchronize on each side.  Graph mode replays a graph
        of `per_graph` consecutive steps (so that one-layer workloads still
        rotate over their KV pools) and a one-step graph for any remainder;
        the captured graph first runs untimed for `warmup` steps and the warm
        time.  Events between replays give the spread of the step time.
        Returns (ms for all steps, per-step ms of each replay, host s)."""
        import torch
        if self.eager:
            chunks = [(lambda k=k: one_step(warmup + k), 1) for k in range(steps)]
        else:
            full, rem = divmod(steps, per_graph)
            chunks = []
            g = self.capture(lambda: [one_step(k) for k in range(per_graph)])
            if full:
                chunks += [(g.replay, per_graph)] * full
            if rem:
                g1 = self.capture(lambda: one_step(0))
                g1.replay()
                chunks += [(g1.replay, 1)] * rem
            a, b = self.events()
            a.record(self.stream)
            g.replay()
            b.record(self.stream)
            b.synchronize()
            per_replay_ms = max(a.elapsed_time(b), 1e-3)
            for _ in range(max(-(-warmup // per_graph),
                               math.ceil(self.next_warm / per_replay_ms))):
                g.replay()
            self.next_warm = self.warm_later
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(chunks) + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record(self.stream)
        for i, (run_chunk, _) in enumerate(chunks):
            run_chunk()
            evs[i + 1].record(self.stream)
        torch.cuda.synchronize()
        host_s = time.perf_counter() - t0
        per = [evs[i].elapsed_time(evs[i + 1]) / n for i, (_, n) in enumerate(chunks)]
        return evs[0].elapsed_time(evs[-1]), per, host_s


def measure(name, args, clock, steps, warmup, layers=None):
    """Time one workload's step (plan once, then decode + combine per layer)
    as two launches per layer and fused, and its kernels on their own.
    Returns (result dict, runner, problem)."""
    import torch

    from load_balanced_split_amd import runner, workloads as wl

    note("measuring", name)
    w = wl.WORKLOADS[name]
    multi_layer = w.layers > 1
    if layers is None:
        layers = args.layers if args.layers is not None else (w.layers if multi_layer else 1)
    pools = layers if multi_layer else max(1, args.pools)
    prob = wl.make_problem(name, seed=args.seed, device="cuda", layers=pools)
    run = runner.DecodeRunner(prob, num_bins=args.num_bins, min_tiles=args.min_tiles)
    live_tokens = int(prob.seq_lens.sum())
    kv_bytes_layer = live_tokens * wl.kv_bytes_per_token(w)

    def step(k):
        """One decode step: plan once, then decode + combine per layer."""
        run.plan()
        for layer in range(layers):
            run.decode((k * layers + layer) % pools)
            run.combine()

    def fused_step(k):
        """The same step with decode and combine in one launch per layer."""
        run.plan()
        for layer in range(layers):
            run.decode_combine((k * layers + layer) % pools)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    per_graph = 1 if layers >= pools else pools // layers
    total_ms, step_ms, wall = clock.timed(step, steps, warmup, per_graph)
    t_step = total_ms / steps
    total_fused_ms, _, _ = clock.timed(fused_step, steps, warmup, per_graph)
    t_fused = total_fused_ms / steps

    # Per-kernel GPU time, each kernel back to back in its own graph.
    n_dec = max(layers, pools) if multi_layer else pools
    fused_avg = clock.graph_avg_ms(lambda: [run.decode_combine(i % pools) for i in range(n_dec)],
                                   n_dec, warm=clock.warm_later)
    dec_avg = clock.graph_avg_ms(lambda: [run.decode(i % pools) for i in range(n_dec)], n_dec,
                                 warm=clock.warm_later)
    combine_ms = clock.graph_avg_ms(lambda: [run.combine() for _ in range(16)], 16)
    plan_ms = clock.graph_avg_ms(lambda: [run.plan() for _ in range(16)], 16)
    torch.cuda.synchronize()

    value = kv_bytes_layer * layers / (t_step * 1e-3) / 1e9
    achieved = kv_bytes_layer / (dec_avg * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(t_step, 4),
        "us_per_step": round(t_step * 1e3, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if w.kv_dtype == "fp8" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": DESCRIPTIONS[name],
            "batch": int(prob.seq_lens.shape[0]),
            "layers": layers,
            "live_kv_tokens": live_tokens,
            "kv_bytes_per_layer": kv_bytes_layer,
            "num_bins": run.num_bins,
            "min_tiles": run.min_tiles,
            "num_desc": run.num_desc(),
            "seed": args.seed,
            "q_rows": w.q_rows,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        # Each kernel's average comes from its own graph of back-to-back
        # launches, so the residual (step - plan - layers x (decode +
        # combine)) is the launch overhead inside the step minus what the
        # isolated averages over-count; it can come out negative.
        "breakdown_us": {"plan": round(plan_ms * 1e3, 2),
                         "decode_avg": round(dec_avg * 1e3, 2),
                         "combine": round(combine_ms * 1e3, 2),
                         "residual": round((t_step - plan_ms - layers * (dec_avg + combine_ms))
                                           * 1e3, 1),
                         "step_min": round(min(step_ms) * 1e3, 1),
                         "step_p90": round(sorted(step_ms)[int(0.9 * (len(step_ms) - 1))] * 1e3,
                                           1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(name),
                     "kernel": "%s (one launch = one layer's live KV)" % (
                         "decode_shared_kernel" if w.q_rows * w.group > 16 else "decode_kernel")},
        "fused": {"us_per_step": round(t_fused * 1e3, 1),
                  "gbs": round(kv_bytes_layer * layers / (t_fused * 1e-3) / 1e9, 2),
                  "decode_combine_avg_us": round(fused_avg * 1e3, 2),
                  "speedup_vs_two_launches": round(t_step / t_fused, 4)},
        "wall_s_timed": round(wall, 3),
        "launch": "eager" if args.eager else "hip_graph (%d step(s) per replay)" % per_graph,
    }
    res["_layers"], res["_pools"], res["_dec_avg"] = layers, pools, dec_avg
    return res, run, prob


def heavy_tail_orders(args, clock):
    """The heavy-tail batch in its three orders (the 8 long requests at seeded
    random positions, first, last): dynamic decode + combine as two launches
    and fused, against every point of the static split-KV sweep, each as a
    graph of back-to-back calls rotating over the KV pools."""
    import torch

    from load_balanced_split_amd import runner, workloads as wl

    res = {"workload": DESCRIPTIONS["heavy_tail"], "target_speedup_vs_best_static": 1.5}
    for order, name in (("random", "heavy_tail"), ("long_first", "heavy_tail_long_first"),
                        ("long_last", "heavy_tail_long_last")):
        note("heavy-tail order", order, "with the static sweep")
        prob = wl.make_problem(name, seed=args.seed, device="cuda", layers=max(1, args.pools))
        run = runner.DecodeRunner(prob, num_bins=args.num_bins, min_tiles=args.min_tiles)
        sw = static_sweep(run, prob, 1, max(1, args.pools), clock)
        kv = int(prob.seq_lens.sum()) * wl.kv_bytes_per_token(prob.workload)
        sw["kv_gbs_two_launches"] = round(kv / (sw["dynamic_us"] * 1e-6) / 1e9, 1)
        sw["kv_gbs_fused"] = round(kv / (sw["dynamic_fused_us"] * 1e-6) / 1e9, 1)
        res[order] = sw
        del run, prob
        torch.cuda.empty_cache()
    best = max(res["random"]["speedup_vs_best_static"],
               res["random"]["fused_speedup_vs_best_static"])
    res["random_best_speedup"] = best
    res["target_met"] = best >= 1.5
    return res


def shard_step(args, clock):
    """One GPU's head shard of the mixed batch (1 KV head, 8 query heads,
    32 layers): the step timed like the headline's, in a compact record."""
    import torch
    steps = max(5, min(args.steps, 20))
    r, run, prob = measure("mixed_shard", args, clock, steps, min(args.warmup, 5))
    del run, prob
    torch.cuda.empty_cache()
    return {"workload": DESCRIPTIONS["mixed_shard"], "steps": steps,
            "us_per_step": r["us_per_step"], "kv_gbs": r["value"],
            "pct_hbm_peak": r["pct_hbm_peak"], "breakdown_us": r["breakdown_us"],
            "decode_roofline_frac": r["roofline"]["frac"], "fused": r["fused"],
            "num_bins": r["config"]["num_bins"], "num_desc": r["config"]["num_desc"],
            "kv_bytes_per_layer": r["config"]["kv_bytes_per_layer"]}


def main():
    args = parse_args()
    if args.calibrate:
        calibrate()
        return
    if args.oracle_layer:
        oracle_layer(args.workload, args.seed)
        return
    if args.workload == "prologue":
        prologue_bench()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.set_device(0)
    clock = Clock(torch.cuda.current_stream(), args.warm_ms, args.eager)
    out, run, prob = measure(args.workload, args, clock, args.steps, args.warmup)
    layers, pools, dec_avg = out.pop("_layers"), out.pop("_pools"), out.pop("_dec_avg")

    if args.ablation:
        out["ablation"] = static_sweep(run, prob, layers, pools, clock)
    if prob.workload.q_rows > 1:
        out["multi_row"] = rows_as_requests(prob, layers, pools, out["ms_per_step"], dec_avg,
                                            clock, args)
    if not args.no_cpu_baseline:
        note("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(prob, args.cpu_seconds)
    if args.workload == "mixed" and not args.no_extras:
        del run, prob
        torch.cuda.empty_cache()
        out["heavy_tail"] = heavy_tail_orders(args, clock)
        out["mixed_shard"] = shard_step(args, clock)
    print(json.dumps(out), flush=True)


def rows_as_requests(prob, layers, pools, step_ms, dec_ms, clock, args):
    """The same draft-verify step done by a decode that takes one query row
    per request: each of the R rows of request b becomes a request of its own
    over the first L_b - (R - 1 - r) tokens (same page-table row, same KV
    pools, same query bytes), planned and combined as B R requests."""
    import numpy as np

    from load_balanced_split_amd import runner, workloads as wl

    w, R = prob.workload, prob.workload.q_rows
    B = prob.seq_lens.shape[0]
    lens = np.repeat(prob.seq_lens, R) - np.tile(np.arange(R - 1, -1, -1), B)
    one = wl.Workload(w.name + "_rows", None, w.num_kv_heads, w.num_q_heads, w.head_dim,
                      w.kv_dtype, layers=w.layers, num_bins=w.num_bins, min_tiles=w.min_tiles)
    flat = wl.Problem(one, np.maximum(lens, 0).astype(np.int32),
                      np.repeat(prob.page_table, R, axis=0), prob.num_pages,
                      prob.q.view(B * R, w.num_q_heads, w.head_dim), prob.k_pages, prob.v_pages,
                      None if prob.q_scale is None else prob.q_scale.view(B * R, w.num_q_heads),
                      prob.k_scale, prob.v_scale, prob.sm_scale)
    run = runner.DecodeRunner(flat, num_bins=args.num_bins, min_tiles=args.min_tiles)

    def step():
        run.plan()
        for layer in range(layers):
            run.decode(layer % pools)
            run.combine()

    step()
    warm = clock.warm_later   # warmed like the step and decode it is set against
    per = clock.graph_avg_ms(step, 1, reps=max(2, min(10, args.steps)), warm=warm)
    n_dec = max(layers, pools)
    dec = clock.graph_avg_ms(lambda: [run.decode(i % pools) for i in range(n_dec)], n_dec,
                             warm=warm)
    return {"rows": R,
            "rows_as_requests_us_per_step": round(per * 1e3, 1),
            "rows_as_requests_decode_avg_us": round(dec * 1e3, 2),
            "speedup_vs_rows_as_requests": round(per / step_ms, 3),
            "decode_speedup_vs_rows_as_requests": round(dec / dec_ms, 3)}


def static_sweep(run, prob, layers, pools, clock, reps=8):
    """Time the static split-KV baseline (decode + combine) at every sweep
    point against dynamic decode + combine (two launches, and fused) on the
    same pools, each as a HIP graph of `reps` back-to-back calls rotating
    over the pools, replayed untimed for the warm time first."""
    import torch

    def timed(fn):
        fn(0)                       # allocates the sweep point's buffers
        torch.cuda.synchronize()
        g = clock.capture(lambda: [fn((r + 1) % pools) for r in range(reps)])
        a, b = clock.events()
        a.record(clock.stream)
        g.replay()
        b.record(clock.stream)
        b.synchronize()
        for _ in range(math.ceil(clock.warm_later / max(a.elapsed_time(b), 1e-3))):
            g.replay()
        torch.cuda.synchronize()
        a.record(clock.stream)
        for _ in range(5):
            g.replay()
        b.record(clock.stream)
        b.synchronize()
        return a.elapsed_time(b) / (5 * reps) * 1e3

    def dyn(pool):
        run.decode(pool)
        run.combine()

    run.plan()   # one map for every replay (the plan's cost is not in either side)
    torch.cuda.synchronize()
    res = {"dynamic_us": round(timed(dyn), 2),
           "dynamic_fused_us": round(timed(lambda p: run.decode_combine(p)), 2),
           "static_us": {}}
    for S in (1, 2, 4, 8, 16, 32, 64, 128):
        res["static_us"]["splits=%d" % S] = round(timed(lambda p: run.static(0, S, p)), 2)
    for C in (256, 512, 1024, 2048, 4096, 8192):
        res["static_us"]["chunk=%d" % C] = round(timed(lambda p: run.static(1, C, p)), 2)
    run.release_static()
    best = min(res["static_us"], key=res["static_us"].get)
    res["best_static"] = best
    res["best_static_us"] = res["static_us"][best]
    res["speedup_vs_best_static"] = round(res["static_us"][best] / res["dynamic_us"], 3)
    res["fused_speedup_vs_best_static"] = round(res["static_us"][best] / res["dynamic_fused_us"],
                                                3)
    return res


if __name__ == "__main__":
    main()
