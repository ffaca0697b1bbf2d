"""rodimus_scan_prefill_noalloc (the prefill for callers that cannot allocate)
against rodimus_scan_prefill, through the C ABI: two calls in a row, the
second smaller, so the second runs on a scratch array that still holds the
first call's segment states; each must equal the workspace entry point's
result bit for bit (same kernels, same plan) and meet the bf16 bar against the
oracle."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, err, host, log

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "theta")


def _noalloc(d, S0, o, S_T, chunk):
    B, H, T, dk = d["q"].shape
    dv = d["v"].shape[-1]
    p = lambda t: None if t is None else t.data_ptr()
    st = rd.lib().rodimus_scan_prefill_noalloc(*(p(d[n]) for n in NAMES), p(S0), p(o), p(S_T), B, H, T, dk, dv,
                                               chunk, rd.BF16, torch.cuda.current_stream().cuda_stream)
    assert st == rd.OK, rd.status_string(st)


@pytest.mark.parametrize("chunk", [64, 32])
def test_noalloc_prefill_equals_workspace_prefill_two_calls(chunk):
    # first the 1.6B-shaped batch (4 segments of 2 sub-segments per (b,h)),
    # then a smaller one with an initial state and a ragged tail (16 segments)
    cases = [(311, 4, 16, 4096, False), (312, 1, 4, 1000, True)]
    for seed, B, H, T, with_S0 in cases:
        log(f"noalloc prefill: B={B} H={H} T={T} C={chunk} S0={with_S0}")
        x = workloads.scan_inputs(seed, B, H, T, 128, 128, "bf16")
        d = {n: dev(x[n]) for n in NAMES}
        S0 = workloads.device_normal((B, H, 128, 128), seed + 1).float() * 0.5 if with_S0 else None
        assert rd.rodimus_scan_prefill_workspace_bytes(B, H, T, 128, 128, chunk) > 0   # the scratch is used
        o_ref, ST_ref = rd.rodimus_scan_prefill(*(d[n] for n in NAMES), S0, chunk)
        o = torch.full_like(o_ref, float("nan"))
        ST = torch.full_like(ST_ref, float("nan"))
        _noalloc(d, S0, o, ST, chunk)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(ST, ST_ref)
        args = [x[n].f64() for n in NAMES]
        ro, rST = oracle.scan(*args, S0=None if S0 is None else host(S0), nthreads=16)
        eo, es = err(host(o), ro), err(host(ST), rST)
        log(f"  equal to rodimus_scan_prefill; against the oracle: err o {eo:.2e} S_T {es:.2e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
