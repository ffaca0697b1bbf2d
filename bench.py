"""Benchmark of the Rodimus* token-mixer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
                    [--only all|prefill|decode|long|swska|swska_decode|backward|varlen|backward_varlen|copy]

A step is one rodimus_scan_prefill call over the 1.6B-shaped prefill batch
(B=4, T=4096, H=16, dk=dv=128, bf16 inputs, fp32 state, C=64) with every input
already resident in HBM; value = B*T / step time (prefill tokens/s).  The
decode state update (256 sequences x 16 heads, fp32 128x128 states, in-place
steps cycling over 8 resident input sets) is timed in the same run and
reported as HBM GB/s and fraction of peak, as the metric asks.  The
long-context prefill (T=131072), SW-SKA (T=32768, w=4096), the SW-SKA decode
step, the backward of the prefill scan (same 1.6B batch) and a packed
dynamic batch of 64 ragged requests (16384 tokens per head), forward and
backward, are timed as extras.

Timing: W untimed warm-up steps, then K steps between two HIP events on the
stream the kernels run on (torch's current stream), with device syncs on both
sides.  One prefill call launches up to three kernels (segment states, their
combination, the output pass); the roofline entry is for that whole call.

Algorithmic bytes: prefill, per token-head, q, k, g, tau (4 x 256 B) + v (256 B)
in and o (256 B) out = 1536 B, plus the fp32 final state; decode, per head, the
fp32 state read and written (2 x 64 KiB) plus 5 x 256 B of inputs and 256 B of
output; SW-SKA, q, v, o per token-head and the shared k per token; backward,
per token-head, q, k, g, tau, v, dO in (bf16, 6 x 256 B) and dq, dk, dg, dtau,
dv out (fp32, 5 x 512 B) = 4096 B, plus the fp32 dS0.  Peaks: HBM
8 TB/s; dense bf16 MFMA 2.5 PFLOP/s.

"traffic" is the HBM byte count per call measured with rocprofv3 counters
(FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), read from
profiles/traffic.json when that file was taken from the current kernel sources
(same source hash); otherwise null.

The CPU baseline is the fp64 oracle run on the host cores over the whole
prefill workload (the "sample" field says so).  --only selects one workload and
skips the JSON summary line (used under rocprofv3).
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (H16,d128,T4K) + decode state-update HBM GB/s, % roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
NAMES = ("q", "k", "v", "g", "theta")
CSRC = os.path.join(ROOT, "gated_linear_attention_ddts_amd", "csrc")
KERNEL_SOURCES = {
    "prefill": ("scan_mfma.hip", "mfma_common.h", "device_common.h"),
    "decode": ("decode.hip", "device_common.h"),
    "swska": ("swska.hip", "device_common.h"),
    "swska_decode": ("swska_decode.hip", "device_common.h"),
    "backward": ("scan_bwd_mfma.hip", "scan_bwd_body.h", "mfma_common.h", "device_common.h"),
}


def _code_only(text: str) -> str:
    """Source text without comments and whitespace (string literals kept), so
    that editing a comment does not count as changing a kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def source_hash(kind: str) -> str:
    """Hash of the code (comments and whitespace removed) of a kernel's sources."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kind: str):
    """HBM bytes per call from profiles/traffic.json, if taken on these sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(kind):
        return None
    return rec.get("bytes_per_call")


def _dev(t):
    import torch
    if t.dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(t.values)).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.storage().view(np.int16))).cuda().view(torch.bfloat16)


def _time(fn, steps, warmup):
    """Average GPU time (ms) of fn() over `steps` calls, HIP events on torch's stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def prefill_bytes(B, H, T, dk, dv):
    return B * H * T * (4 * dk * 2 + dv * 2 + dv * 2) + B * H * dk * dv * 4


def prefill_flops(B, H, T, dk, dv, C):
    # causal-triangle count: 4 dk dv (state in/out) + (C+1)(dk+dv) intra-chunk per token-head
    return B * H * T * (4 * dk * dv + (C + 1) * (dk + dv))


def bench_prefill(cfg, steps, warmup):
    import torch
    import gated_linear_attention_ddts_amd as rd
    import workloads
    x = workloads.scan_inputs(cfg["seed"], cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"],
                              cfg["dtype"], gate_mu=cfg["gate_mu"])
    d = {n: _dev(x[n]) for n in NAMES}
    del x
    B, H, T, dk, dv, C = cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"], cfg["chunk"]
    o = torch.empty(B, H, T, dv, dtype=d["q"].dtype, device="cuda")
    ST = torch.empty(B, H, dk, dv, dtype=torch.float32, device="cuda")
    nws = rd.rodimus_scan_prefill_workspace_bytes(B, H, T, dk, dv, C, rd.BF16)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def step():
        rd.rodimus_scan_prefill(d["q"], d["k"], d["v"], d["g"], d["theta"], None, C, o=o, S_T=ST,
                                workspace=ws)

    ms = _time(step, steps, warmup)
    nbytes = prefill_bytes(B, H, T, dk, dv)
    flops = prefill_flops(B, H, T, dk, dv, C)
    return dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), bytes=nbytes, flops=flops,
                gbs=nbytes / (ms * 1e-3) / 1e9, tflops=flops / (ms * 1e-3) / 1e12,
                workspace_bytes=nws)


def bench_varlen(cfg, steps, warmup):
    import torch
    import gated_linear_attention_ddts_amd as rd
    import workloads
    N, H, total, dk, dv, C = cfg["N"], cfg["H"], cfg["total"], cfg["dk"], cfg["dv"], cfg["chunk"]
    L = workloads.ragged_lengths(cfg["seed"], N, total, cfg["min_len"])
    x = workloads.packed_scan_inputs(cfg["seed"], H, total, dk, dv, cfg["dtype"])
    d = {n: _dev(x[n]) for n in NAMES}
    del x
    cu = torch.from_numpy(workloads.cu_seqlens(L)).cuda()
    maxlen = int(L.max())
    o = torch.empty(H, total, dv, dtype=d["q"].dtype, device="cuda")
    ST = torch.empty(N, H, dk, dv, dtype=torch.float32, device="cuda")
    nws = rd.rodimus_scan_prefill_varlen_workspace_bytes(N, H, maxlen, dk, dv, C, rd.BF16)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def step():
        rd.rodimus_scan_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["theta"], cu, maxlen, None, C, o=o,
                                       S_T=ST, workspace=ws)

    ms = _time(step, steps, warmup)
    # per token-head q, k, g, tau, v in and o out (bf16), plus every fp32 S_T
    nbytes = H * total * (4 * dk * 2 + dv * 2 + dv * 2) + N * H * dk * dv * 4
    return dict(ms=ms, tokens_per_s=total / (ms * 1e-3), bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
                sequences=N, max_len=maxlen, min_len=int(L.min()))


def bench_backward_varlen(cfg, steps, warmup):
    import torch
    import gated_linear_attention_ddts_amd as rd
    import workloads
    N, H, total, dk, dv = cfg["N"], cfg["H"], cfg["total"], cfg["dk"], cfg["dv"]
    L = workloads.ragged_lengths(cfg["seed"], N, total, cfg["min_len"])
    x = workloads.packed_scan_inputs(cfg["seed"], H, total, dk, dv, cfg["dtype"])
    d = {n: _dev(x[n]) for n in NAMES}
    del x
    dO = workloads.device_normal((H, total, dv), cfg["seed"] + 1000)
    cu = torch.from_numpy(workloads.cu_seqlens(L)).cuda()
    maxlen = int(L.max())
    ws = torch.empty(rd.rodimus_scan_backward_varlen_workspace_bytes(N, H, maxlen, dk, dv, rd.BF16),
                     dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = dict(dq=torch.empty(H, total, dk, **f32), dk=torch.empty(H, total, dk, **f32),
               dv=torch.empty(H, total, dv, **f32), dg=torch.empty(H, total, dk, **f32),
               dtau=torch.empty(H, total, dk, **f32), dS0=torch.empty(N, H, dk, dv, **f32))

    def step():
        rd.rodimus_scan_backward_varlen(d["q"], d["k"], d["v"], d["g"], d["theta"], dO, cu, maxlen, out=out,
                                        workspace=ws)

    ms = _time(step, steps, warmup)
    # per token-head the same bytes as the batched backward, plus every fp32 dS0
    nbytes = backward_bytes(1, H, total, dk, dv) - H * dk * dv * 4 + N * H * dk * dv * 4
    return dict(ms=ms, tokens_per_s=total / (ms * 1e-3), bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
                sequences=N, max_len=maxlen, min_len=int(L.min()), workspace_bytes=ws.numel())


def backward_bytes(B, H, T, dk, dv):
    # in: q, k, g, tau, v, dO (bf16); out: dq, dk, dg, dtau, dv (fp32); plus dS0 (fp32)
    return B * H * T * ((4 * dk + 2 * dv) * 2 + (4 * dk + dv) * 4) + B * H * dk * dv * 4


def backward_flops(B, H, T, dk, dv, C=32):
    # per token-head: five dk x dv products (state checkpoint, state gradient,
    # S dO^T, G v^T, Kb G) and the causal-triangle intra-chunk terms (dP, A,
    # dq, dk over dk or dv channels, dv over dv)
    return B * H * T * (10 * dk * dv + (C + 1) * (3 * dk + 2 * dv))


def bench_backward(cfg, steps, warmup):
    import torch
    import gated_linear_attention_ddts_amd as rd
    import workloads
    B, H, T, dk, dv = cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"]
    x = workloads.scan_inputs(cfg["seed"], B, H, T, dk, dv, cfg["dtype"], gate_mu=cfg["gate_mu"])
    d = {n: _dev(x[n]) for n in NAMES}
    del x
    dO = workloads.device_normal((B, H, T, dv), cfg["seed"] + 1000)
    ws = torch.empty(rd.rodimus_scan_backward_workspace_bytes(B, H, T, dk, dv, rd.BF16),
                     dtype=torch.uint8, device="cuda")

    def step():
        # the binding allocates the five gradient tensors per call from torch's
        # caching allocator (no device synchronisation)
        rd.rodimus_scan_backward(d["q"], d["k"], d["v"], d["g"], d["theta"], dO, workspace=ws)

    ms = _time(step, steps, warmup)
    nbytes = backward_bytes(B, H, T, dk, dv)
    flops = backward_flops(B, H, T, dk, dv)
    return dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), bytes=nbytes, flops=flops,
                gbs=nbytes / (ms * 1e-3) / 1e9, tflops=flops / (ms * 1e-3) / 1e12,
                workspace_bytes=ws.numel())


def decode_bytes(N, H, dk, dv):
    return N * H * (2 * dk * dv * 4 + (4 * dk + dv) * 2 + dv * 2)


def bench_decode(cfg, steps, warmup):
    import torch
    import gated_linear_attention_ddts_amd as rd
    import workloads
    N, H, dk, dv = cfg["N"], cfg["H"], cfg["dk"], cfg["dv"]
    sets = workloads.decode_pool(cfg["seed"], N, H, dk, dv, pool=cfg["pool"], dtype=cfg["dtype"])
    dsets = [{n: _dev(s[n]) for n in NAMES} for s in sets]
    S = torch.zeros(N, H, dk, dv, dtype=torch.float32, device="cuda")
    o = torch.empty(N, H, dv, dtype=torch.bfloat16, device="cuda")
    state = {"s": 0}

    def step():
        s = dsets[state["s"] % len(dsets)]
        state["s"] += 1
        rd.rodimus_decode_step(s["q"], s["k"], s["v"], s["g"], s["theta"], S, o=o)

    ms = _time(step, steps, warmup)
    ms_graph = _graph_time(step, len(dsets), 8)

    # ping-pong: S_in and S_out alternate between two buffers, so the step
    # reads one 268 MB state and writes another (a 537 MB working set, twice the
    # 256 MB Infinity Cache) instead of updating one in place
    S2 = torch.zeros_like(S)

    def step_pp():
        s = dsets[state["s"] % len(dsets)]
        a, b = (S, S2) if state["s"] % 2 == 0 else (S2, S)
        state["s"] += 1
        rd.rodimus_decode_step(s["q"], s["k"], s["v"], s["g"], s["theta"], a, b, o=o)

    ms_pp = _time(step_pp, steps, warmup)
    nbytes = decode_bytes(N, H, dk, dv)
    return dict(ms=ms, us_per_step=ms * 1e3, tokens_per_s=N / (ms * 1e-3), bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9, steps=steps, us_per_step_graph=ms_graph * 1e3,
                us_per_step_pingpong=ms_pp * 1e3, gbs_pingpong=nbytes / (ms_pp * 1e-3) / 1e9)


def _graph_time(step, n_capture, replays):
    """Per-step GPU time (ms) of `step` captured n_capture times into one HIP
    graph and replayed: what a serving loop without per-step launches sees."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(n_capture):
            step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n_capture):
            step()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * n_capture)


def swska_pairs(T, w):
    # query-key pairs inside the causal band: sum_t min(t+1, w)
    n = min(T, w)
    return n * (n + 1) // 2 + (T - n) * w


def bench_swska(cfg, steps, warmup):
    import torch
    import gated_linear_attention_ddts_amd as rd
    import workloads
    B, H, T, dk, dv, w = cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"], cfg["window"]
    x = workloads.swska_inputs(cfg["seed"], B, H, T, dk, dv)
    d = {n: _dev(x[n]) for n in ("q", "k", "v")}
    o = torch.empty(B, H, T, dv, dtype=torch.bfloat16, device="cuda")

    def step():
        rd.sw_ska_attn(d["q"], d["k"], d["v"], w, o=o)

    ms = _time(step, steps, warmup)
    flops = B * H * swska_pairs(T, w) * 2 * (dk + dv)
    nbytes = (B * H * T * (dk + 2 * dv) + B * T * dk) * 2
    return dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), flops=flops,
                tflops=flops / (ms * 1e-3) / 1e12, bytes=nbytes)


def swska_decode_bytes(N, H, dk, dv, window):
    # per sequence-step: the shared key window and every head's value window read;
    # q, k_new, v_new read; the new key/values written to the caches; o written (bf16)
    return N * (window * dk * 2 + H * window * dv * 2 + H * dk * 2 + 2 * (dk * 2 + H * dv * 2)
                + H * dv * 2)


def bench_swska_decode(cfg, steps, warmup):
    """Decode steps over full window caches; each step appends one token per
    sequence (the library advances the positions)."""
    import torch
    import gated_linear_attention_ddts_amd as rd
    import workloads
    N, H, dk, dv, W = cfg["N"], cfg["H"], cfg["dk"], cfg["dv"], cfg["window"]
    kc = workloads.device_normal((N, W, dk), cfg["seed"] * 100 + 1)
    vc = workloads.device_normal((N, H, W, dv), cfg["seed"] * 100 + 2)
    pool = workloads.swska_inputs(cfg["seed"], N, H, cfg["pool"], dk, dv)
    qs, ks, vs = (_dev(pool[n]) for n in ("q", "k", "v"))
    toks = [(qs[:, :, i].contiguous(), ks[:, i].contiguous(), vs[:, :, i].contiguous())
            for i in range(cfg["pool"])]
    pos = torch.full((N,), cfg["pos0"], dtype=torch.int32, device="cuda")
    o = torch.empty(N, H, dv, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(rd.sw_ska_decode_workspace_bytes(N, H, dk, dv, W), dtype=torch.uint8,
                     device="cuda")
    state = {"s": 0}

    def step():
        qn, kn, vn = toks[state["s"] % len(toks)]
        state["s"] += 1
        rd.sw_ska_decode_step(qn, kn, vn, kc, vc, pos, o=o, workspace=ws)

    ms = _time(step, steps, warmup)
    ms_graph = _graph_time(step, len(toks), 4)
    nbytes = swska_decode_bytes(N, H, dk, dv, W)
    return dict(ms=ms, us_per_step=ms * 1e3, tokens_per_s=N / (ms * 1e-3), bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9, steps=steps, us_per_step_graph=ms_graph * 1e3)


def bench_copy(nbytes=1 << 30, steps=5):
    """A plain device-to-device copy of known size (counter calibration)."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    ms = _time(lambda: b.copy_(a), steps, 1)
    return dict(ms=ms, read_bytes=a.numel(), write_bytes=b.numel(),
                gbs=2 * a.numel() / (ms * 1e-3) / 1e9)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, min_cpu_s=12.0, max_reps=40):
    """The fp64 oracle on the host cores over the whole prefill workload, repeated
    until the process has spent at least min_cpu_s seconds of CPU time (all
    threads together); the rate is the mean over the repetitions.  Also timed
    single-threaded (the plain sequential definition) on one (b,h) pair."""
    import oracle
    import workloads
    nproc = os.cpu_count() or 1
    cores = min(nproc, 16)
    x = workloads.scan_inputs(cfg["seed"], cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"],
                              cfg["dtype"], gate_mu=cfg["gate_mu"])
    arrs = [x[n].f64() for n in NAMES]
    del x
    reps = 0
    c0, t0 = time.process_time(), time.perf_counter()
    while reps < max_reps:
        oracle.scan(*arrs, nthreads=cores)
        reps += 1
        if time.process_time() - c0 >= min_cpu_s:
            break
    dt = time.perf_counter() - t0
    cpu = time.process_time() - c0
    one = [np.ascontiguousarray(a[:1, :1]) for a in arrs]
    t1 = time.perf_counter()
    oracle.scan(*one, nthreads=1)
    dt1 = time.perf_counter() - t1
    BT = cfg["B"] * cfg["T"]
    return dict(value=round(reps * BT / dt, 1), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"the whole workload (B={cfg['B']} x T={cfg['T']} tokens x H={cfg['H']} heads, "
                       f"fp64 sequential scan per (b,h) on {cores} threads) run {reps} times: "
                       f"{dt:.2f} s wall, {cpu:.1f} s CPU",
                single_thread=dict(value=round(cfg["T"] / dt1 / cfg["H"], 1), unit="tokens/s",
                                   sample=f"one (b,h) pair of T={cfg['T']} tokens on 1 thread, "
                                          f"{dt1:.3f} s; tokens/s counts a token as all {cfg['H']} heads"),
                nproc=nproc, cpu_model=_cpu_model())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="all", choices=["all", "prefill", "decode", "long", "swska", "swska_decode", "backward", "varlen",
                             "backward_varlen", "copy"])
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not run here. Every (b,h) pair, "
              "sequence and head is independent, so N GPUs would each run this same workload on "
              "their own share (weak scaling).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.only != "all":
        if args.only == "prefill":
            r = bench_prefill(workloads.CONFIGS["prefill_1p6b_T4096"], args.steps, args.warmup)
        elif args.only == "long":
            r = bench_prefill(workloads.CONFIGS["prefill_long_T131072"], args.steps, args.warmup)
        elif args.only == "decode":
            r = bench_decode(workloads.CONFIGS["decode_N256"], args.steps, args.warmup)
        elif args.only == "swska":
            r = bench_swska(workloads.CONFIGS["swska_T32768_w4096"], args.steps, args.warmup)
        elif args.only == "swska_decode":
            r = bench_swska_decode(workloads.CONFIGS["swska_decode_N64_w4096"], args.steps, args.warmup)
        elif args.only == "backward":
            r = bench_backward(workloads.CONFIGS["prefill_1p6b_T4096"], args.steps, args.warmup)
        elif args.only == "varlen":
            r = bench_varlen(workloads.CONFIGS["prefill_varlen_N64_16K"], args.steps, args.warmup)
        elif args.only == "backward_varlen":
            r = bench_backward_varlen(workloads.CONFIGS["prefill_varlen_N64_16K"], args.steps, args.warmup)
        else:
            r = bench_copy()
        print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}),
              flush=True)
        return

    cfg = workloads.CONFIGS["prefill_1p6b_T4096"]
    print("bench: prefill_1p6b_T4096", file=sys.stderr, flush=True)
    pre = bench_prefill(cfg, args.steps, args.warmup)
    print("bench: decode_N256", file=sys.stderr, flush=True)
    dec = bench_decode(workloads.CONFIGS["decode_N256"], args.decode_steps, 10)
    print("bench: prefill_long_T131072", file=sys.stderr, flush=True)
    lc = workloads.CONFIGS["prefill_long_T131072"]
    lr = bench_prefill(lc, max(3, args.steps // 4), 1)
    print("bench: swska_T32768_w4096", file=sys.stderr, flush=True)
    sr = bench_swska(workloads.CONFIGS["swska_T32768_w4096"], max(3, args.steps // 4), 1)
    print("bench: swska_decode_N64_w4096", file=sys.stderr, flush=True)
    sdc = workloads.CONFIGS["swska_decode_N64_w4096"]
    sd = bench_swska_decode(sdc, sdc["steps"], 10)
    print("bench: backward_1p6b_T4096", file=sys.stderr, flush=True)
    bw = bench_backward(cfg, max(5, args.steps // 2), 2)
    print("bench: prefill_varlen_N64_16K", file=sys.stderr, flush=True)
    vl = bench_varlen(workloads.CONFIGS["prefill_varlen_N64_16K"], args.steps, args.warmup)
    print("bench: backward_varlen_N64_16K", file=sys.stderr, flush=True)
    bvl = bench_backward_varlen(workloads.CONFIGS["prefill_varlen_N64_16K"], max(5, args.steps // 2), 2)

    cpu = None
    if not args.no_cpu:
        print("bench: cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg)

    tr = measured_traffic("prefill_1p6b_T4096", "prefill")
    dtr = measured_traffic("decode_N256", "decode")
    line = {
        "metric": METRIC,
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_1p6b_T4096", "B": cfg["B"], "T": cfg["T"], "H": cfg["H"],
                   "dk": cfg["dk"], "dv": cfg["dv"], "chunk": cfg["chunk"],
                   "state_dtype": "fp32"},
        "roofline": {"bound": "hbm", "achieved": round(pre["gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(pre["gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": tr, "kernel": "rodimus_scan_prefill call (segment states + "
                     "combine + output pass)", "algorithmic_bytes": pre["bytes"],
                     "mfma_frac": round(pre["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)},
        "cpu_baseline": cpu,
        "decode": {"workload": "decode_N256", "us_per_step": round(dec["us_per_step"], 2),
                   "us_per_step_graph": round(dec["us_per_step_graph"], 2),
                   "us_per_step_pingpong": round(dec["us_per_step_pingpong"], 2),
                   "frac_pingpong": round(dec["gbs_pingpong"] / HBM_PEAK_GBS, 4),
                   "tokens_per_s": round(dec["tokens_per_s"]), "steps": dec["steps"],
                   "roofline": {"bound": "hbm", "achieved": round(dec["gbs"], 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(dec["gbs"] / HBM_PEAK_GBS, 4), "traffic": dtr,
                                "kernel": "decode_step_kernel<bf16,128,128>",
                                "algorithmic_bytes": dec["bytes"]}},
        "extras": {
            "prefill_long_T131072": {
                "ms": round(lr["ms"], 4), "tokens_per_s": round(lr["tokens_per_s"]),
                "roofline": {"bound": "hbm", "achieved": round(lr["gbs"], 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(lr["gbs"] / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic("prefill_long_T131072", "prefill"),
                             "algorithmic_bytes": lr["bytes"]}},
            "swska_T32768_w4096": {
                "ms": round(sr["ms"], 4), "tokens_per_s": round(sr["tokens_per_s"]),
                "roofline": {"bound": "mfma", "achieved": round(sr["tflops"], 1),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(sr["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                             "traffic": measured_traffic("swska_T32768_w4096", "swska"),
                             "algorithmic_bytes": sr["bytes"]}},
            "swska_decode_N64_w4096": {
                "us_per_step": round(sd["us_per_step"], 2), "tokens_per_s": round(sd["tokens_per_s"]),
                "us_per_step_graph": round(sd["us_per_step_graph"], 2),
                "steps": sd["steps"],
                "roofline": {"bound": "hbm", "achieved": round(sd["gbs"], 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(sd["gbs"] / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic("swska_decode_N64_w4096", "swska_decode"),
                             "algorithmic_bytes": sd["bytes"]}},
            "backward_1p6b_T4096": {
                "ms": round(bw["ms"], 4), "tokens_per_s": round(bw["tokens_per_s"]),
                "roofline": {"bound": "hbm", "achieved": round(bw["gbs"], 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(bw["gbs"] / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic("backward_1p6b_T4096", "backward"),
                             "kernel": "rodimus_scan_backward call (state passes + combine + "
                             "gradients + fallback)", "algorithmic_bytes": bw["bytes"],
                             "workspace_bytes": bw["workspace_bytes"]}},
            "prefill_varlen_N64_16K": {
                "ms": round(vl["ms"], 4), "tokens_per_s": round(vl["tokens_per_s"]),
                "sequences": vl["sequences"], "min_len": vl["min_len"], "max_len": vl["max_len"],
                "roofline": {"bound": "hbm", "achieved": round(vl["gbs"], 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(vl["gbs"] / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic("prefill_varlen_N64_16K", "prefill"),
                             "algorithmic_bytes": vl["bytes"]}},
            "backward_varlen_N64_16K": {
                "ms": round(bvl["ms"], 4), "tokens_per_s": round(bvl["tokens_per_s"]),
                "sequences": bvl["sequences"], "min_len": bvl["min_len"], "max_len": bvl["max_len"],
                "roofline": {"bound": "hbm", "achieved": round(bvl["gbs"], 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(bvl["gbs"] / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic("backward_varlen_N64_16K", "backward"),
                             "algorithmic_bytes": bvl["bytes"], "workspace_bytes": bvl["workspace_bytes"]}},
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
