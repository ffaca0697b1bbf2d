"""Concurrent calls on separate streams.  The library keeps no mutable global
state and takes all scratch from the caller's workspace, so calls on different
streams (with their own workspaces and outputs), issued from different host
threads, must give exactly what the same calls give one after the other on
the current stream.  Streams are created at the default priority."""
import threading

import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import workloads
from tests.gpu_helpers import dev, log

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "theta")


def _prefill_job(seed):
    B, H, T, d = 1, 8, 1500, 128
    x = workloads.scan_inputs(seed, B, H, T, d, d, "bf16")
    dd = {n: dev(x[n]) for n in NAMES}
    ws = torch.empty(rd.rodimus_scan_prefill_workspace_bytes(B, H, T, d, d, 64), dtype=torch.uint8, device="cuda")
    return lambda stream=None: rd.rodimus_scan_prefill(*(dd[n] for n in NAMES), None, 64, workspace=ws,
                                                       stream=stream)


def _backward_job(seed):
    B, H, T, d = 1, 4, 900, 128
    x = workloads.scan_inputs(seed, B, H, T, d, d, "bf16")
    dd = {n: dev(x[n]) for n in NAMES}
    dO = workloads.device_normal((B, H, T, d), seed + 1)
    ws = torch.empty(rd.rodimus_scan_backward_workspace_bytes(B, H, T, d, d), dtype=torch.uint8, device="cuda")
    return lambda stream=None: rd.rodimus_scan_backward(*(dd[n] for n in NAMES), dO, workspace=ws, stream=stream)


def _decode_job(seed):
    N, H, d, K = 32, 8, 128, 5
    sets = workloads.decode_pool(seed, N, H, d, d, pool=K)
    dsets = [{n: dev(s[n]) for n in NAMES} for s in sets]
    S0 = workloads.device_normal((N, H, d, d), seed + 1).float()

    def run(stream=None):
        S = S0.clone()
        outs = [rd.rodimus_decode_step(*(dsets[i][n] for n in NAMES), S, stream=stream) for i in range(K)]
        return S, outs
    return run


def _flat(r):
    if isinstance(r, dict):
        return [r[k] for k in sorted(r) if r[k] is not None]
    if isinstance(r, tuple):
        out = []
        for x in r:
            out += x if isinstance(x, list) else ([x] if x is not None else [])
        return out
    return [r]


def test_concurrent_streams_from_two_host_threads():
    jobs = [_prefill_job(120), _backward_job(122), _decode_job(124), _prefill_job(126)]
    ref = [_flat(j()) for j in jobs]                  # one after the other, current stream
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in jobs]     # default priority
    res = [None] * len(jobs)

    def worker(idx):
        for i in idx:
            with torch.cuda.stream(streams[i]):
                res[i] = _flat(jobs[i](streams[i]))
    threads = [threading.Thread(target=worker, args=([0, 2],)), threading.Thread(target=worker, args=([1, 3],))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, res)):
        assert len(a) == len(b)
        for x, y in zip(a, b):
            assert torch.equal(x, y), i
    log(f"  {len(jobs)} jobs on {len(streams)} streams from 2 threads: bit for bit as run in sequence")
