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
sides and no event between the steps (an event between two kernels costs about
10 us here).  The per-call median and minimum come from a separate run of
batches of calls, each batch between two events and at least 1 ms long.  One
prefill call launches up to three kernels (segment states, their combination,
the output pass); the roofline entry is for that whole call.

A GPU that has just been idle runs the first tens of milliseconds of any load
below the clock it holds under sustained load (at W = 5 the headline comes out
about 10% slower, SW-SKA about 25%).  So the headline's W warm-up steps are
preceded by about 200 ms of a neutral load, bf16 matrix products on torch (the
"precondition" field), and the same K steps timed before it are reported as
"clock_rising".  Every other workload warms up on its own calls for at least
200 ms ("warmup_calls").

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
import math
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
    "prefill": ("scan_mfma.hip", "scan_state.hip", "scan_mfma.h", "mfma_common.h", "device_common.h"),
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
    """Hash of the code (comments and whitespace removed) of a kernel's sources
    and of their per-file compiler options."""
    from gated_linear_attention_ddts_amd.build import FILE_FLAGS
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
        if f in FILE_FLAGS:   # compiler options change the code too
            h.update(" ".join(FILE_FLAGS[f]).encode())
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


LAST_TIMING = {}


def _time(fn, steps, warmup, settle_ms=0.0):
    """Average GPU time (ms) of fn() over `steps` back-to-back calls between two
    HIP events on torch's stream (the stream the library launches on).
    Untimed warm-up first: `warmup` calls, then, with `settle_ms`, more calls
    until that much wall time has passed since the first (the count is kept as
    warmup_calls).  An event recorded between two calls costs about 10 us on
    this GPU (it waits for the queue and writes back the caches), so none sits
    inside the timed run; the per-call median and minimum come from a second
    run of min(steps, 50) batches, each of enough calls to last 1 ms or more
    between its two events, and are kept in LAST_TIMING beside the mean."""
    import torch
    t0 = time.perf_counter()
    n = 0
    for _ in range(warmup):
        fn()
        n += 1
    if settle_ms > 0:
        torch.cuda.synchronize()
        while (time.perf_counter() - t0) * 1e3 < settle_ms:
            for _ in range(8):
                fn()
            n += 8
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / steps
    reps = max(1, math.ceil(1.0 / max(mean, 1e-3)))
    nb = min(steps, 50)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    ev[0].record()
    for i in range(nb):
        for _ in range(reps):
            fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) / reps for i in range(nb)]
    LAST_TIMING.clear()
    LAST_TIMING.update(mean=mean, median=float(np.median(per)), min=float(np.min(per)), warmup_calls=n,
                       spread_batches=nb, spread_calls_per_batch=reps)
    return mean


# Untimed warm-up of each extra workload: its own calls for this long.  A GPU
# that has just been idle (process start, host-side input generation between
# workloads) runs the first tens of milliseconds of any load below the clock it
# holds under sustained load.
SETTLE_MS = 200.0


def _precondition(ms=200.0, n=4096):
    """Brings the GPU to its sustained operating point before the headline's
    warm-up steps without running the headline workload itself: a bf16 matrix
    product of two n x n matrices (torch), repeated for `ms` of wall time after
    one untimed call that initialises the library.  A memory-bound load (a
    device fill) leaves the graphics clock lower, and the prefill's gate map,
    which runs on the vector ALUs, then starts about 4% slower.  Returns
    (ms, products)."""
    import torch
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    a @ a
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    k = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            a @ a
        k += 8
        torch.cuda.synchronize()
    del a
    return (time.perf_counter() - t0) * 1e3, k


def _time_cold(fn, steps, flush_bytes=512 << 20):
    """Per-call GPU time (ms) with the caches cold: before each call a
    `flush_bytes` buffer (twice the 256 MB Infinity Cache) is written, and only
    the call itself sits between the two events.  Returns (median, min)."""
    import torch
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    per = []
    for i in range(steps):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    del flush
    return float(np.median(per)), float(np.min(per))


def _timing_fields(ms_scale=1.0, prefix="ms"):
    t = dict(LAST_TIMING)
    return {f"{prefix}_median": round(t["median"] * ms_scale, 4), f"{prefix}_min": round(t["min"] * ms_scale, 4),
            "warmup_calls": t["warmup_calls"],
            "median_min_over": f"{t['spread_batches']} batches of {t['spread_calls_per_batch']} calls"}


def prefill_bytes(B, H, T, dk, dv):
    return B * H * T * (4 * dk * 2 + dv * 2 + dv * 2) + B * H * dk * dv * 4


def prefill_flops(B, H, T, dk, dv, C):
    # causal-triangle count: 4 dk dv (state in/out) + (C+1)(dk+dv) intra-chunk per token-head
    return B * H * T * (4 * dk * dv + (C + 1) * (dk + dv))


def bench_prefill(cfg, steps, warmup, cold=True, headline=False):
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

    extra = {}
    if headline:
        # exactly `warmup` untimed calls before the `steps` timed ones.  First as
        # the process comes up (the clock still rising: reported, not the
        # figure), then again after a neutral load has brought the GPU to its
        # sustained operating point (the figure)
        ms_cc = _time(step, steps, warmup)
        tf_cc = _timing_fields()
        pre_ms, pre_n = _precondition()
        ms = _time(step, steps, warmup)
        extra = dict(clock_rising=dict(ms=round(ms_cc, 4), **tf_cc),
                     precondition=dict(ms=round(pre_ms, 1), products=pre_n,
                                       what="4096 x 4096 bf16 matrix products (torch) repeated, before the "
                                            "warm-up steps"))
    else:
        ms = _time(step, steps, warmup, settle_ms=SETTLE_MS)
    tf = _timing_fields()
    cold_med, cold_min = _time_cold(step, max(5, steps // 2)) if cold else (None, None)
    nbytes = prefill_bytes(B, H, T, dk, dv)
    flops = prefill_flops(B, H, T, dk, dv, C)
    r = dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), bytes=nbytes, flops=flops,
             gbs=nbytes / (ms * 1e-3) / 1e9, tflops=flops / (ms * 1e-3) / 1e12,
             workspace_bytes=nws, **tf, **extra)
    if cold:
        r.update(ms_cold_median=cold_med, ms_cold_min=cold_min,
                 gbs_cold=nbytes / (cold_med * 1e-3) / 1e9)
    return r


def lowrank_bytes(B, H, T, dk, dv, R):
    # q, k, v in and o out (bf16) per token-head; the factor rows per token
    # (shared by the heads); the per-head factors and biases; the fp32 S_T
    return (B * H * T * (2 * dk + dv + dv) * 2 + B * T * 2 * R * 2 + H * (2 * dk * R * 2 + 2 * dk * 4)
            + B * H * dk * dv * 4)


def bench_lowrank(cfg, steps, warmup, bias_sigma=None):
    """The 1.6B-shaped prefill with the gate logits expanded in-kernel from
    rank-R factor rows (g and tau never stored).  bias_sigma overrides the
    workload's bias spread (random biases give some channels a decay fast
    enough to send a few chunks to the token-by-token fallback)."""
    import torch
    import gated_linear_attention_ddts_amd as rd
    import workloads
    B, H, T, dk, dv, C, R = cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"], cfg["chunk"], cfg["R"]
    bs = cfg["bias_sigma"] if bias_sigma is None else bias_sigma
    x = workloads.lowrank_inputs(cfg["seed"], B, H, T, dk, dv, R, bias_sigma=bs)
    names = ("q", "k", "v", "zg", "zt", "Ug", "bg", "Ut", "bt")
    d = {n: _dev(x[n]) for n in names}
    del x
    o = torch.empty(B, H, T, dv, dtype=torch.bfloat16, device="cuda")
    ST = torch.empty(B, H, dk, dv, dtype=torch.float32, device="cuda")
    nws = rd.rodimus_scan_prefill_workspace_bytes(B, H, T, dk, dv, C, rd.BF16)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")

    def step():
        rd.rodimus_scan_prefill_lowrank(*(d[n] for n in names), None, C, o=o, S_T=ST, workspace=ws)

    ms = _time(step, steps, warmup, settle_ms=SETTLE_MS)
    tf = _timing_fields()
    nbytes = lowrank_bytes(B, H, T, dk, dv, R)
    return dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
                bytes_per_token_head=nbytes / (B * H * T), **tf)


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

    ms = _time(step, steps, warmup, settle_ms=SETTLE_MS)
    # per token-head q, k, g, tau, v in and o out (bf16), plus every fp32 S_T
    nbytes = H * total * (4 * dk * 2 + dv * 2 + dv * 2) + N * H * dk * dv * 4
    return dict(ms=ms, tokens_per_s=total / (ms * 1e-3), bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
                sequences=N, max_len=maxlen, min_len=int(L.min()), **_timing_fields())


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

    ms = _time(step, steps, warmup, settle_ms=SETTLE_MS)
    # per token-head the same bytes as the batched backward, plus every fp32 dS0
    nbytes = backward_bytes(1, H, total, dk, dv) - H * dk * dv * 4 + N * H * dk * dv * 4
    return dict(ms=ms, tokens_per_s=total / (ms * 1e-3), bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
                sequences=N, max_len=maxlen, min_len=int(L.min()), workspace_bytes=ws.numel(),
                **_timing_fields())


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

    ms = _time(step, steps, warmup, settle_ms=SETTLE_MS)
    nbytes = backward_bytes(B, H, T, dk, dv)
    flops = backward_flops(B, H, T, dk, dv)
    return dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), bytes=nbytes, flops=flops,
                gbs=nbytes / (ms * 1e-3) / 1e9, tflops=flops / (ms * 1e-3) / 1e12,
                workspace_bytes=ws.numel(), **_timing_fields())


def decode_bytes(N, H, dk, dv):
    return N * H * (2 * dk * dv * 4 + (4 * dk + dv) * 2 + dv * 2)


def bench_decode(cfg, steps, warmup, big_n=1024):
    """Decode steps on resident states, three ways:
    * in place, N = 256: the workload as specified; its 268 MB state is about
      the size of the 256 MB Infinity Cache, so part of each step is served
      from that cache (cache-assisted, labelled so);
    * ping-pong, N = 256: S_in and S_out alternate between two buffers, so each
      step reads one 268 MB state and writes another (a 537 MB working set):
      the HBM-true rate of the same step, and the roofline figure;
    * in place, N = `big_n`: a 1.07 GB state, far larger than the cache."""
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

    ms = _time(step, steps, warmup, settle_ms=SETTLE_MS)
    tf = _timing_fields(1e3, "us_per_step")
    ms_graph = _graph_time(step, len(dsets), 8)

    S2 = torch.zeros_like(S)

    def step_pp():
        s = dsets[state["s"] % len(dsets)]
        a, b = (S, S2) if state["s"] % 2 == 0 else (S2, S)
        state["s"] += 1
        rd.rodimus_decode_step(s["q"], s["k"], s["v"], s["g"], s["theta"], a, b, o=o)

    ms_pp = _time(step_pp, steps, warmup, settle_ms=SETTLE_MS)
    tf_pp = _timing_fields(1e3, "us_per_step")
    del S2

    # a batch whose state is four times the cache: inputs replicated from the pool
    rep = big_n // N
    bsets = [{n: t.repeat(rep, *([1] * (t.dim() - 1))).contiguous() for n, t in s.items()} for s in dsets]
    Sb = torch.zeros(big_n, H, dk, dv, dtype=torch.float32, device="cuda")
    ob = torch.empty(big_n, H, dv, dtype=torch.bfloat16, device="cuda")

    def step_big():
        s = bsets[state["s"] % len(bsets)]
        state["s"] += 1
        rd.rodimus_decode_step(s["q"], s["k"], s["v"], s["g"], s["theta"], Sb, o=ob)

    ms_big = _time(step_big, max(50, steps // 4), warmup, settle_ms=SETTLE_MS)
    tf_big = _timing_fields(1e3, "us_per_step")
    del Sb, bsets
    nbytes = decode_bytes(N, H, dk, dv)
    nbig = decode_bytes(big_n, H, dk, dv)
    return dict(ms=ms, us_per_step=ms * 1e3, tokens_per_s=N / (ms * 1e-3), bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9, steps=steps, us_per_step_graph=ms_graph * 1e3,
                timing=tf, us_per_step_pingpong=ms_pp * 1e3, gbs_pingpong=nbytes / (ms_pp * 1e-3) / 1e9,
                timing_pingpong=tf_pp, tokens_per_s_pingpong=N / (ms_pp * 1e-3),
                big_n=big_n, us_per_step_big=ms_big * 1e3, bytes_big=nbig,
                gbs_big=nbig / (ms_big * 1e-3) / 1e9, timing_big=tf_big)


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

    ms = _time(step, steps, warmup, settle_ms=SETTLE_MS)
    flops = B * H * swska_pairs(T, w) * 2 * (dk + dv)
    nbytes = (B * H * T * (dk + 2 * dv) + B * T * dk) * 2
    return dict(ms=ms, tokens_per_s=B * T / (ms * 1e-3), flops=flops,
                tflops=flops / (ms * 1e-3) / 1e12, bytes=nbytes, **_timing_fields())


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

    ms = _time(step, steps, warmup, settle_ms=SETTLE_MS)
    tf = _timing_fields(1e3, "us_per_step")
    ms_graph = _graph_time(step, len(toks), 4)
    nbytes = swska_decode_bytes(N, H, dk, dv, W)
    return dict(ms=ms, us_per_step=ms * 1e3, tokens_per_s=N / (ms * 1e-3), bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9, steps=steps, us_per_step_graph=ms_graph * 1e3, **tf)


def bench_mixer_chain(N=16, H=16, d=128, window=4096, layers=2, pos0=8192, steps=200, warmup=10, seed=8):
    """Rodimus+ decode at a small batch: per token, in each of `layers` layers,
    a Rodimus decode step then an SW-SKA decode step over a full window cache,
    each mixer's output being the next one's query (the projections between
    them are outside this library).  Timed eagerly (one launch after another)
    and replayed from one HIP graph holding 8 tokens' launches."""
    import torch
    import gated_linear_attention_ddts_amd as rd
    import workloads
    pool = 8
    rsets = [workloads.decode_pool(seed * 10 + l, N, H, d, d, pool=pool) for l in range(layers)]
    r_in = [[{n: _dev(x[n]) for n in NAMES} for x in rsets[l]] for l in range(layers)]
    sx = [workloads.swska_inputs(seed * 10 + 5 + l, N, H, pool, d, d) for l in range(layers)]
    s_in = [[(_dev(sx[l]["k"])[:, i].contiguous(), _dev(sx[l]["v"])[:, :, i].contiguous()) for i in range(pool)]
            for l in range(layers)]
    S = [torch.zeros(N, H, d, d, device="cuda") for _ in range(layers)]
    kc = [workloads.device_normal((N, window, d), seed * 100 + l) for l in range(layers)]
    vc = [workloads.device_normal((N, H, window, d), seed * 100 + 50 + l) for l in range(layers)]
    pos = [torch.full((N,), pos0, dtype=torch.int32, device="cuda") for _ in range(layers)]
    ws = [torch.empty(rd.sw_ska_decode_workspace_bytes(N, H, d, d, window), dtype=torch.uint8, device="cuda")
          for _ in range(layers)]
    o_r = [torch.empty(N, H, d, dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    o_s = [torch.empty(N, H, d, dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    state = {"s": 0}

    def step():
        i = state["s"] % pool
        state["s"] += 1
        q = r_in[0][i]["q"]
        for l in range(layers):
            x = r_in[l][i]
            rd.rodimus_decode_step(q, x["k"], x["v"], x["g"], x["theta"], S[l], o=o_r[l])
            rd.sw_ska_decode_step(o_r[l], *s_in[l][i], kc[l], vc[l], pos[l], o=o_s[l], workspace=ws[l])
            q = o_s[l]

    ms = _time(step, steps, warmup, settle_ms=SETTLE_MS)
    tf = _timing_fields(1e3, "us_per_token")
    ms_graph = _graph_time(step, pool, max(4, steps // pool))
    nbytes = layers * (decode_bytes(N, H, d, d) + swska_decode_bytes(N, H, d, d, window))
    return dict(us_per_token=ms * 1e3, us_per_token_graph=ms_graph * 1e3, tokens_per_s=N / (ms * 1e-3),
                tokens_per_s_graph=N / (ms_graph * 1e-3), bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
                gbs_graph=nbytes / (ms_graph * 1e-3) / 1e9, launches_per_token=3 * layers, **tf,
                config=dict(N=N, H=H, d=d, window=window, layers=layers))


def bench_stream(nbytes, steps=50):
    """A plain device-to-device copy (torch's copy kernel, no arithmetic) of
    nbytes into a second buffer: the read+write rate of a pure stream of the
    same size as the decode step's state, measured the same way."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    ms = _time(lambda: b.copy_(a), steps, 5, settle_ms=SETTLE_MS)
    return dict(us=ms * 1e3, gbs=2 * nbytes / (ms * 1e-3) / 1e9, **_timing_fields(1e3, "us"))


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


def _oracle_cores():
    return min(os.cpu_count() or 1, 16)


def cpu_baseline_long(cfg, T_sample=16384):
    """The oracle on every head of the long-context prefill over its first
    T_sample tokens (the per-token cost of the sequential recurrence does not
    depend on the position), one head per thread."""
    import oracle
    import workloads
    cores = _oracle_cores()
    x = workloads.scan_inputs(cfg["seed"], cfg["B"], cfg["H"], T_sample, cfg["dk"], cfg["dv"], cfg["dtype"],
                              gate_mu=cfg["gate_mu"])
    arrs = [x[n].f64() for n in NAMES]
    del x
    c0, t0 = time.process_time(), time.perf_counter()
    oracle.scan(*arrs, nthreads=cores)
    dt, cpu = time.perf_counter() - t0, time.process_time() - c0
    return dict(value=round(cfg["B"] * T_sample / dt, 1), unit="tokens/s", cores=min(cores, cfg["B"] * cfg["H"]),
                kind="oracle",
                sample=f"all {cfg['H']} heads over the first {T_sample} of the {cfg['T']} tokens (inputs drawn "
                       f"with the workload's recipe at that length), fp64 sequential scan, one (b,h) per thread: "
                       f"{dt:.2f} s wall, {cpu:.1f} s CPU")


def cpu_baseline_backward(cfg, T_sample=1024):
    """The oracle's backward (the gradients of the sequential recurrence, fp64 C
    loops, one (b,h) per thread) on every head of the first sequence over its
    first T_sample tokens."""
    import oracle
    import workloads
    cores = _oracle_cores()
    H, dk, dv = cfg["H"], cfg["dk"], cfg["dv"]
    x = workloads.scan_inputs(cfg["seed"], 1, H, T_sample, dk, dv, cfg["dtype"], gate_mu=cfg["gate_mu"])
    arrs = [x[n].f64() for n in NAMES]
    del x
    dO = np.random.default_rng(cfg["seed"] + 1000).standard_normal((1, H, T_sample, dv))
    c0, t0 = time.process_time(), time.perf_counter()
    oracle.scan_backward(*arrs, dO, nthreads=cores)
    dt, cpu = time.perf_counter() - t0, time.process_time() - c0
    return dict(value=round(T_sample / dt, 1), unit="tokens/s", cores=min(cores, H), kind="oracle",
                sample=f"all {H} heads of one sequence over its first {T_sample} of the {cfg['T']} tokens, "
                       f"fp64 gradients of the sequential recurrence, one (b,h) per thread: {dt:.2f} s wall, "
                       f"{cpu:.1f} s CPU; a token is all {H} heads")


def cpu_baseline_decode(cfg, steps=6):
    """The oracle's decode step (single-threaded C loop) over the whole batch of
    N sequences x H heads, for `steps` steps from zero states."""
    import oracle
    import workloads
    sets = workloads.decode_pool(cfg["seed"], cfg["N"], cfg["H"], cfg["dk"], cfg["dv"], pool=cfg["pool"],
                                 dtype=cfg["dtype"])
    S = np.zeros((cfg["N"], cfg["H"], cfg["dk"], cfg["dv"]))
    xs = [[s[n].f64() for n in NAMES] for s in sets]
    c0, t0 = time.process_time(), time.perf_counter()
    for i in range(steps):
        _, S = oracle.decode(*xs[i % len(xs)], S)
    dt, cpu = time.perf_counter() - t0, time.process_time() - c0
    return dict(value=round(steps * cfg["N"] / dt, 1), unit="tokens/s", cores=1, kind="oracle",
                sample=f"{steps} steps of the whole {cfg['N']}-sequence x {cfg['H']}-head batch (fp64 states "
                       f"{cfg['dk']}x{cfg['dv']}), single-threaded: {dt:.2f} s wall, {cpu:.1f} s CPU; "
                       f"us per step {dt / steps * 1e6:.0f}")


def cpu_baseline_swska(cfg, rows_per_head=128):
    """The oracle's dense softmax per query row on rows_per_head rows of every
    head, spread over the part of the sequence where the window is full."""
    import oracle
    import workloads
    cores = _oracle_cores()
    B, H, T, D, w = cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["window"]
    x = workloads.swska_inputs(cfg["seed"], B, H, T, D, D)
    ts = np.linspace(w, T - 1, rows_per_head).astype(np.int64)
    rows = (np.arange(H)[:, None] * T + ts[None, :]).reshape(-1)
    q, k, v = (x[n].f64() for n in ("q", "k", "v"))
    del x
    c0, t0 = time.process_time(), time.perf_counter()
    oracle.swska(q, k, v, w, rows=rows, nthreads=cores)
    dt, cpu = time.perf_counter() - t0, time.process_time() - c0
    # a token is all H heads' rows
    return dict(value=round(rows.size / H / dt, 1), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{rows_per_head} query rows per head x {H} heads with a full {w}-key window, "
                       f"fp64 dense softmax per row on {cores} threads: {dt:.2f} s wall, {cpu:.1f} s CPU")


def _rl(bound, achieved, peak, unit, traffic, nbytes, **extra):
    d = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic, "algorithmic_bytes": nbytes}
    d.update(extra)
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="all", choices=["all", "prefill", "decode", "long", "swska", "swska_decode",
                                                      "backward", "varlen", "backward_varlen", "lowrank", "chain",
                                                      "stream", "copy"])
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
            r = bench_prefill(workloads.CONFIGS["prefill_1p6b_T4096"], args.steps, args.warmup, cold=False)
        elif args.only == "long":
            r = bench_prefill(workloads.CONFIGS["prefill_long_T131072"], args.steps, args.warmup, cold=False)
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
        elif args.only == "lowrank":
            r = bench_lowrank(workloads.CONFIGS["prefill_lowrank_1p6b_T4096"], args.steps, args.warmup)
        elif args.only == "stream":
            c = workloads.CONFIGS["decode_N256"]
            r = bench_stream(c["N"] * c["H"] * c["dk"] * c["dv"] * 4, args.steps)
        elif args.only == "chain":
            r = bench_mixer_chain(steps=args.steps, warmup=args.warmup)
        else:
            r = bench_copy()
        print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}),
              flush=True)
        return

    def stage(name):
        print(f"bench: {name}", file=sys.stderr, flush=True)

    cfg = workloads.CONFIGS["prefill_1p6b_T4096"]
    stage("prefill_1p6b_T4096")
    pre = bench_prefill(cfg, args.steps, args.warmup, headline=True)
    stage("decode_N256")
    dec = bench_decode(workloads.CONFIGS["decode_N256"], args.decode_steps, 10)
    dc = workloads.CONFIGS["decode_N256"]
    stm = bench_stream(dc["N"] * dc["H"] * dc["dk"] * dc["dv"] * 4)
    stm_big = bench_stream(dec["big_n"] * dc["H"] * dc["dk"] * dc["dv"] * 4, 20)
    stage("prefill_long_T131072")
    lc = workloads.CONFIGS["prefill_long_T131072"]
    lr = bench_prefill(lc, max(3, args.steps // 4), 1)
    stage("swska_T32768_w4096")
    sc = workloads.CONFIGS["swska_T32768_w4096"]
    sr = bench_swska(sc, max(3, args.steps // 4), 1)
    stage("swska_decode_N64_w4096")
    sdc = workloads.CONFIGS["swska_decode_N64_w4096"]
    sd = bench_swska_decode(sdc, sdc["steps"], 10)
    stage("rodimus_plus_decode_2layer_N16")
    ch = bench_mixer_chain()
    stage("prefill_lowrank_1p6b_T4096")
    lrc = workloads.CONFIGS["prefill_lowrank_1p6b_T4096"]
    lrk = bench_lowrank(lrc, args.steps, args.warmup)
    lrk_rb = bench_lowrank(lrc, args.steps, args.warmup, bias_sigma=0.5)
    stage("backward_1p6b_T4096")
    bw = bench_backward(cfg, max(5, args.steps // 2), 2)
    stage("prefill_varlen_N64_16K")
    vl = bench_varlen(workloads.CONFIGS["prefill_varlen_N64_16K"], args.steps, args.warmup)
    stage("backward_varlen_N64_16K")
    bvl = bench_backward_varlen(workloads.CONFIGS["prefill_varlen_N64_16K"], max(5, args.steps // 2), 2)

    cpu = cpu_long = cpu_dec = cpu_ska = cpu_bwd = None
    if not args.no_cpu:
        stage("cpu baselines (fp64 oracle)")
        cpu = cpu_baseline(cfg)
        cpu_long = cpu_baseline_long(lc)
        cpu_dec = cpu_baseline_decode(workloads.CONFIGS["decode_N256"])
        cpu_ska = cpu_baseline_swska(sc)
        cpu_bwd = cpu_baseline_backward(cfg)

    tr = measured_traffic("prefill_1p6b_T4096", "prefill")
    dtr = measured_traffic("decode_N256", "decode")
    dtr_pp = measured_traffic("decode_N256_pingpong", "decode")
    line = {
        "metric": METRIC,
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 4),
        "ms_per_step_median": pre["ms_median"],
        "ms_per_step_min": pre["ms_min"],
        "clock_rising": pre["clock_rising"],
        "precondition": pre["precondition"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_1p6b_T4096", "B": cfg["B"], "T": cfg["T"], "H": cfg["H"],
                   "dk": cfg["dk"], "dv": cfg["dv"], "chunk": cfg["chunk"],
                   "state_dtype": "fp32"},
        "roofline": _rl("hbm", pre["gbs"], HBM_PEAK_GBS, "GB/s", tr, pre["bytes"],
                        kernel="rodimus_scan_prefill call (segment states + output pass with the incoming states folded in)",
                        mfma_frac=round(pre["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                        cold_cache={"ms_median": round(pre["ms_cold_median"], 4),
                                    "ms_min": round(pre["ms_cold_min"], 4),
                                    "achieved": round(pre["gbs_cold"], 1),
                                    "frac": round(pre["gbs_cold"] / HBM_PEAK_GBS, 4),
                                    "how": "512 MB written before each call; events around the call only"}),
        "cpu_baseline": cpu,
        "decode": {
            "workload": "decode_N256", "steps": dec["steps"],
            "us_per_step": round(dec["us_per_step_pingpong"], 2),
            "tokens_per_s": round(dec["tokens_per_s_pingpong"]),
            **dec["timing_pingpong"],
            "roofline": _rl("hbm", dec["gbs_pingpong"], HBM_PEAK_GBS, "GB/s", dtr_pp, dec["bytes"],
                            kernel="decode_step_kernel<bf16,128,128> (streaming state loads)",
                            working_set="S_in and S_out alternate between two 268 MB buffers (537 MB, "
                                        "twice the 256 MB Infinity Cache): HBM-true"),
            "in_place_cache_assisted": {
                "us_per_step": round(dec["us_per_step"], 2), **dec["timing"],
                "us_per_step_graph": round(dec["us_per_step_graph"], 2),
                "tokens_per_s": round(dec["tokens_per_s"]),
                "achieved": round(dec["gbs"], 1), "frac": round(dec["gbs"] / HBM_PEAK_GBS, 4),
                "traffic": dtr,
                "note": "state updated in place; the 268 MB state is about the 256 MB Infinity Cache's size, "
                        "so part of each step is served from that cache"},
            f"in_place_N{dec['big_n']}": {
                "us_per_step": round(dec["us_per_step_big"], 2), **dec["timing_big"],
                "achieved": round(dec["gbs_big"], 1), "frac": round(dec["gbs_big"] / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": dec["bytes_big"],
                "note": f"{dec['big_n']} sequences: a {dec['big_n'] * 16 * 65536 / 1e9:.2f} GB state updated in "
                        "place, far larger than the cache: HBM-true"},
            "stream_copy_same_bytes": {
                "us": round(stm["us"], 2), "us_median": stm["us_median"], "us_min": stm["us_min"],
                "achieved": round(stm["gbs"], 1), "frac": round(stm["gbs"] / HBM_PEAK_GBS, 4),
                "note": "a plain device copy (no arithmetic) of one 268 MB buffer into another: the "
                        "read+write streaming rate of the ping-pong step's bytes"},
            f"stream_copy_N{dec['big_n']}_bytes": {
                "us": round(stm_big["us"], 2), "achieved": round(stm_big["gbs"], 1),
                "frac": round(stm_big["gbs"] / HBM_PEAK_GBS, 4),
                "note": f"the same copy at the {dec['big_n']}-sequence state's size, far beyond the cache"},
            "cpu_baseline": cpu_dec},
        "extras": {
            "prefill_long_T131072": {
                "ms": round(lr["ms"], 4), "ms_median": lr["ms_median"], "ms_min": lr["ms_min"],
                "tokens_per_s": round(lr["tokens_per_s"]),
                "roofline": _rl("hbm", lr["gbs"], HBM_PEAK_GBS, "GB/s",
                                measured_traffic("prefill_long_T131072", "prefill"), lr["bytes"],
                                cold_cache={"ms_median": round(lr["ms_cold_median"], 4),
                                            "frac": round(lr["gbs_cold"] / HBM_PEAK_GBS, 4)}),
                "cpu_baseline": cpu_long},
            "swska_T32768_w4096": {
                "ms": round(sr["ms"], 4), "ms_median": sr["ms_median"], "ms_min": sr["ms_min"],
                "tokens_per_s": round(sr["tokens_per_s"]),
                "roofline": _rl("mfma", sr["tflops"], MFMA_BF16_PEAK_TFLOPS, "TFLOP/s",
                                measured_traffic("swska_T32768_w4096", "swska"), sr["bytes"]),
                "cpu_baseline": cpu_ska},
            "swska_decode_N64_w4096": {
                "us_per_step": round(sd["us_per_step"], 2), "us_per_step_median": sd["us_per_step_median"],
                "us_per_step_min": sd["us_per_step_min"], "tokens_per_s": round(sd["tokens_per_s"]),
                "us_per_step_graph": round(sd["us_per_step_graph"], 2),
                "steps": sd["steps"],
                "roofline": _rl("hbm", sd["gbs"], HBM_PEAK_GBS, "GB/s",
                                measured_traffic("swska_decode_N64_w4096", "swska_decode"), sd["bytes"],
                                working_set="1.14 GB of window caches per step: HBM-true"),
                "cpu_baseline": None if cpu_ska is None else dict(
                    cpu_ska, sample="the SW-SKA rows above: a decode token of one sequence is one full-window "
                                    "row per head, the same oracle work")},
            "rodimus_plus_decode_2layer_N16": {
                "us_per_token": round(ch["us_per_token"], 2), "us_per_token_median": ch["us_per_token_median"],
                "us_per_token_min": ch["us_per_token_min"],
                "us_per_token_graph": round(ch["us_per_token_graph"], 2),
                "tokens_per_s": round(ch["tokens_per_s"]), "tokens_per_s_graph": round(ch["tokens_per_s_graph"]),
                "launches_per_token": ch["launches_per_token"], "config": ch["config"],
                "roofline": _rl("hbm", ch["gbs"], HBM_PEAK_GBS, "GB/s", None, ch["bytes"],
                                graph_frac=round(ch["gbs_graph"] / HBM_PEAK_GBS, 4))},
            "prefill_lowrank_1p6b_T4096": {
                "ms": round(lrk["ms"], 4), "ms_median": lrk["ms_median"], "ms_min": lrk["ms_min"],
                "tokens_per_s": round(lrk["tokens_per_s"]),
                "bytes_per_token_head": round(lrk["bytes_per_token_head"], 1),
                "vs_logit_input_prefill": round(pre["ms"] / lrk["ms"], 3),
                "ms_random_biases": round(lrk_rb["ms"], 4),
                "roofline": _rl("hbm", lrk["gbs"], HBM_PEAK_GBS, "GB/s",
                                measured_traffic("prefill_lowrank_1p6b_T4096", "prefill"), lrk["bytes"],
                                kernel="rodimus_scan_prefill_lowrank call (segment states + "
                                       "output pass, gate logits from rank-16 factors in-kernel)")},
            "backward_1p6b_T4096": {
                "ms": round(bw["ms"], 4), "ms_median": bw["ms_median"], "ms_min": bw["ms_min"],
                "tokens_per_s": round(bw["tokens_per_s"]),
                "roofline": _rl("hbm", bw["gbs"], HBM_PEAK_GBS, "GB/s",
                                measured_traffic("backward_1p6b_T4096", "backward"), bw["bytes"],
                                kernel="rodimus_scan_backward call (state passes + combine + gradients + fallback)",
                                workspace_bytes=bw["workspace_bytes"]),
                "cpu_baseline": cpu_bwd},
            "prefill_varlen_N64_16K": {
                "ms": round(vl["ms"], 4), "ms_median": vl["ms_median"], "ms_min": vl["ms_min"],
                "tokens_per_s": round(vl["tokens_per_s"]),
                "sequences": vl["sequences"], "min_len": vl["min_len"], "max_len": vl["max_len"],
                "roofline": _rl("hbm", vl["gbs"], HBM_PEAK_GBS, "GB/s",
                                measured_traffic("prefill_varlen_N64_16K", "prefill"), vl["bytes"])},
            "backward_varlen_N64_16K": {
                "ms": round(bvl["ms"], 4), "ms_median": bvl["ms_median"], "ms_min": bvl["ms_min"],
                "tokens_per_s": round(bvl["tokens_per_s"]),
                "sequences": bvl["sequences"], "min_len": bvl["min_len"], "max_len": bvl["max_len"],
                "roofline": _rl("hbm", bvl["gbs"], HBM_PEAK_GBS, "GB/s",
                                measured_traffic("backward_varlen_N64_16K", "backward"), bvl["bytes"],
                                workspace_bytes=bvl["workspace_bytes"])},
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
