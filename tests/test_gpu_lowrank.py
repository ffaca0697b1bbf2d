"""GPU parity of rodimus_scan_prefill_lowrank (gate logits expanded inside the
kernels from rank-16 factor rows shared by the heads) against the fp64 oracle
(oracle.scan_lowrank: the logits from the factors, then the sequential
recurrence), at the bf16 bar: one and several segments, ragged tails, an
initial state, both chunk sizes, slow decay, chunks that take the token-by-token
fallback, and the 1.6B-shaped batch in full."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, errs, fmt, host, log

pytestmark = pytest.mark.gpu

GPU_NAMES = ("q", "k", "v", "zg", "zt", "Ug", "bg", "Ut", "bt")


def run(x, chunk, S0=None):
    d = {n: dev(x[n]) for n in GPU_NAMES}
    o, ST = rd.rodimus_scan_prefill_lowrank(*(d[n] for n in GPU_NAMES), S0=S0, chunk=chunk)
    torch.cuda.synchronize()
    return host(o), host(ST)


def ref(x, S0=None):
    return oracle.scan_lowrank(*(x[n].f64() for n in GPU_NAMES), S0=None if S0 is None else host(S0), nthreads=16)


def check(x, chunk, S0=None, label=""):
    o, ST = run(x, chunk, S0)
    ro, rST = ref(x, S0)
    eo, es = errs(o, ro), errs(ST, rST)
    log(f"lowrank {label} C={chunk}")
    log(fmt("o", eo))
    log(fmt("S_T", es))
    assert eo["err"] <= TOL["bf16"] and es["err"] <= TOL["bf16"]
    return eo, es


@pytest.mark.parametrize("chunk", [64, 32])
@pytest.mark.parametrize("B,H,T", [(1, 2, 150), (2, 8, 1000), (1, 1, 64), (1, 3, 1), (3, 5, 333)])
def test_lowrank_shapes(B, H, T, chunk):
    x = workloads.lowrank_inputs(400 + T, B, H, T, 128, 128)
    check(x, chunk, label=f"B={B} H={H} T={T}")


def test_lowrank_with_initial_state():
    B, H, T = 2, 4, 700
    x = workloads.lowrank_inputs(410, B, H, T, 128, 128)
    S0 = workloads.device_normal((B, H, 128, 128), 411).float() * 0.5
    check(x, 64, S0, label="S0")


def test_lowrank_slow_decay_long_carry():
    # biases g ~ +4, tau ~ -2: a ~ 0.998 per token, so the state carries far
    B, H, T = 1, 4, 3000
    x = workloads.lowrank_inputs(420, B, H, T, 128, 128, gbias_mu=4.0, tbias_mu=-2.0, bias_sigma=0.3)
    check(x, 64, label="slow decay")


def test_lowrank_every_chunk_takes_the_fallback():
    # g ~ -12, tau ~ +3: log2 a ~ -16 per token, far beyond the factorised
    # form's 2^112 span inside any chunk, so every chunk runs token by token
    B, H, T = 1, 2, 300
    x = workloads.lowrank_inputs(430, B, H, T, 128, 128, gbias_mu=-12.0, tbias_mu=3.0, bias_sigma=0.2)
    check(x, 64, label="fallback everywhere")
    check(x, 32, label="fallback everywhere")


def test_lowrank_stretch_of_fast_decay():
    # selection factor rows of 40 tokens set large: their logits spread with
    # sd ~ 6, so some channels decay fast enough to send those chunks to the
    # fallback while the rest of the sequence takes the matrix-core path
    B, H, T = 1, 4, 900
    x = workloads.lowrank_inputs(440, B, H, T, 128, 128)
    zg = x["zg"].values.copy()
    zg[:, 300:340] = 6.0
    x["zg"] = workloads.Tensor(workloads.round_to(zg, "bf16"), "bf16")
    check(x, 64, label="fast-decay stretch")


def test_lowrank_1p6b_T4096_full_parity():
    c = workloads.CONFIGS["prefill_lowrank_1p6b_T4096"]
    log("prefill_lowrank_1p6b_T4096: inputs")
    x = workloads.lowrank_inputs(c["seed"], c["B"], c["H"], c["T"], c["dk"], c["dv"], c["R"])
    eo, es = check(x, c["chunk"], label="1.6B batch")
    assert eo["per_unit"] <= TOL["bf16"] and es["per_unit"] <= TOL["bf16"]


def test_lowrank_deterministic_and_workspace_shared_with_prefill():
    B, H, T = 2, 8, 777
    x = workloads.lowrank_inputs(450, B, H, T, 128, 128)
    d = {n: dev(x[n]) for n in GPU_NAMES}
    need = rd.rodimus_scan_prefill_workspace_bytes(B, H, T, 128, 128, 64)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1, s1 = rd.rodimus_scan_prefill_lowrank(*(d[n] for n in GPU_NAMES), workspace=ws)
    o2, s2 = rd.rodimus_scan_prefill_lowrank(*(d[n] for n in GPU_NAMES), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    with pytest.raises(rd.RodimusError):
        rd.rodimus_scan_prefill_lowrank(*(d[n] for n in GPU_NAMES), workspace=ws[: need - 16])
