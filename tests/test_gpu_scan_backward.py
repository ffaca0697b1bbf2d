"""GPU parity of rodimus_scan_backward against the oracle's backward (fp64,
reverse-mode through the sequential definition; pinned by finite
differences, autograd of an independent recurrence and closed forms).

Two paths: the generic one (fp32 inputs, or head sizes other than 128)
computes in fp32 from the exact input values and is held to 1e-4; the
matrix-core one (bf16, dk = dv = 128) uses bf16 operands with fp32
accumulation and bf16 state checkpoints, and is held to the bf16 bar (2e-2).
Its cases cover several checkpoint segments (the fix-up of every checkpoint by
the segment's incoming state), one segment, ragged lengths around the 32- and
64-token boundaries, and decays too fast for the factored operands (the exact
fallback), alone and mixed with ordinary halves."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, err, host, log

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "theta")
GRADS = ("dq", "dk", "dv", "dg", "dtau", "dS0")
BWD_TOL = 1e-4


def _tol(dtype, dk, dv):
    return TOL["bf16"] if (dtype == "bf16" and dk == 128 and dv == 128) else BWD_TOL


def _run(x, dO, S0=None, dST=None):
    d = {n: dev(x[n]) for n in NAMES}
    S0d = None if S0 is None else torch.from_numpy(S0.astype(np.float32)).cuda()
    dSTd = None if dST is None else torch.from_numpy(dST.astype(np.float32)).cuda()
    out = rd.rodimus_scan_backward(d["q"], d["k"], d["v"], d["g"], d["theta"], dev(dO), S0d, dSTd)
    torch.cuda.synchronize()
    ref = oracle.scan_backward(*(x[n].f64() for n in NAMES), dO.f64(),
                               None if S0 is None else S0.astype(np.float32).astype(np.float64),
                               None if dST is None else dST.astype(np.float32).astype(np.float64),
                               nthreads=8)
    ref["dtau"] = ref.pop("dtheta")
    return out, ref


def _check(out, ref, tol, label):
    errs = {k: err(host(out[k]), ref[k]) for k in GRADS if out[k] is not None}
    log(f"  {label}: " + " ".join(f"{k} {e:.2e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= tol, (label, k, e)


def _dO(seed, B, H, T, dv, dtype):
    rng = np.random.default_rng(seed)
    return workloads.Tensor(workloads.round_to(rng.standard_normal((B, H, T, dv)), dtype), dtype)


@pytest.mark.parametrize("dtype,B,H,T,dk,dv", [
    ("fp32", 1, 2, 100, 16, 32),
    ("fp32", 2, 1, 77, 48, 80),
    ("bf16", 1, 2, 150, 128, 128),
    ("bf16", 2, 3, 33, 64, 128),
    ("fp32", 1, 1, 70, 128, 128),
    ("bf16", 1, 3, 200, 128, 128),     # three (b,h): many segments
    ("bf16", 2, 2, 1000, 128, 128),
])
def test_backward_shapes(dtype, B, H, T, dk, dv):
    x = workloads.scan_inputs(201, B, H, T, dk, dv, dtype)
    rng = np.random.default_rng(202)
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    dST = rng.standard_normal((B, H, dk, dv)) * 0.5
    out, ref = _run(x, _dO(203, B, H, T, dv, dtype), S0, dST)
    _check(out, ref, _tol(dtype, dk, dv), f"{dtype} B{B} H{H} T{T} dk{dk} dv{dv}")


@pytest.mark.parametrize("T", [1, 31, 32, 33, 64, 95])
def test_backward_ragged_lengths_without_states(T):
    x = workloads.scan_inputs(210 + T, 1, 2, T, 32, 32, "bf16")
    out, ref = _run(x, _dO(211, 1, 2, T, 32, "bf16"))
    _check(out, ref, _tol("bf16", 32, 32), f"T{T}")


@pytest.mark.parametrize("T", [1, 31, 32, 33, 63, 64, 65, 96, 127, 129])
def test_backward_matrix_core_ragged(T):
    x = workloads.scan_inputs(250 + T, 1, 2, T, 128, 128, "bf16")
    rng = np.random.default_rng(251)
    S0 = rng.standard_normal((1, 2, 128, 128)) * 0.5
    dST = rng.standard_normal((1, 2, 128, 128)) * 0.5
    out, ref = _run(x, _dO(252, 1, 2, T, 128, "bf16"), S0, dST)
    _check(out, ref, TOL["bf16"], f"mfma T{T}")


def test_backward_matrix_core_one_segment():
    # 256 (b,h) pairs: the state passes need no segments and no fix-ups
    B, H, T = 64, 4, 160
    x = workloads.scan_inputs(260, B, H, T, 128, 128, "bf16")
    dO = _dO(261, B, H, T, 128, "bf16")
    d = {n: dev(x[n]) for n in NAMES}
    out = rd.rodimus_scan_backward(d["q"], d["k"], d["v"], d["g"], d["theta"], dev(dO))
    torch.cuda.synchronize()
    for b, h in ((0, 0), (37, 2), (63, 3)):
        sub = [x[n].values[b:b + 1, h:h + 1].astype(np.float64) for n in NAMES]
        ref = oracle.scan_backward(*sub, dO.values[b:b + 1, h:h + 1].astype(np.float64))
        ref["dtau"] = ref.pop("dtheta")
        _check({kk: out[kk][b:b + 1, h:h + 1] for kk in GRADS}, ref, TOL["bf16"], f"one segment ({b},{h})")


@pytest.mark.parametrize("where", ["all", "middle"])
def test_backward_matrix_core_fast_decay_fallback(where):
    # gate logits ~ -10 with tau ~ 1: log2 a ~ -14 per token, far past the
    # factored operands' span inside 32 tokens; "middle" makes only some
    # halves take the exact path
    B, H, T = 1, 2, 200
    x = workloads.scan_inputs(270, B, H, T, 128, 128, "bf16")
    lo, hi = (0, T) if where == "all" else (70, 110)
    x["g"].values[:, :, lo:hi] = workloads.round_to(x["g"].values[:, :, lo:hi] - 10.0, "bf16")
    x["theta"].values[:, :, lo:hi] = workloads.round_to(np.abs(x["theta"].values[:, :, lo:hi]) + 3.0, "bf16")
    rng = np.random.default_rng(271)
    S0 = rng.standard_normal((B, H, 128, 128)) * 0.5
    dST = rng.standard_normal((B, H, 128, 128)) * 0.5
    out, ref = _run(x, _dO(272, B, H, T, 128, "bf16"), S0, dST)
    _check(out, ref, TOL["bf16"], f"fallback {where}")


def test_backward_extreme_and_slow_gates():
    # gate logits up to |8| (decays from ~1 to ~3e-4 per token) and a slow-decay head
    B, H, T, dk, dv = 1, 2, 130, 64, 64
    x = workloads.scan_inputs(220, B, H, T, dk, dv, "fp32", gate_sigma=4.0)
    x["g"].values[:, 1] = workloads.round_to(np.full((T, dk), 4.0) + 0.1 * np.arange(dk), "fp32")
    x["theta"].values[:, 1] = -2.0
    out, ref = _run(x, _dO(221, B, H, T, dv, "fp32"))
    _check(out, ref, BWD_TOL, "extreme/slow gates")


def test_backward_linear_attention_limit():
    B, H, T, dk, dv = 1, 2, 70, 32, 16
    x = workloads.scan_inputs(230, B, H, T, dk, dv, "fp32")
    x["theta"].values[:] = -np.inf
    out, ref = _run(x, _dO(231, B, H, T, dv, "fp32"))
    _check(out, ref, BWD_TOL, "tau = 0")
    assert torch.count_nonzero(out["dg"]) == 0 and torch.count_nonzero(out["dtau"]) == 0


def test_backward_empty_sequence_passes_the_state_gradient():
    B, H, dk, dv = 2, 2, 32, 32
    z = torch.empty(B, H, 0, dk, dtype=torch.bfloat16, device="cuda")
    dST = torch.randn(B, H, dk, dv, device="cuda")
    out = rd.rodimus_scan_backward(z, z, torch.empty(B, H, 0, dv, dtype=torch.bfloat16, device="cuda"), z, z,
                                   torch.empty(B, H, 0, dv, dtype=torch.bfloat16, device="cuda"), None, dST)
    torch.cuda.synchronize()
    assert torch.equal(out["dS0"], dST)


def test_backward_prefill_1p6b_T4096_sampled_heads():
    c = workloads.CONFIGS["prefill_1p6b_T4096"]
    B, H, T, dk, dv = c["B"], c["H"], c["T"], c["dk"], c["dv"]
    log("backward T4096: inputs")
    x = workloads.scan_inputs(c["seed"], B, H, T, dk, dv, c["dtype"])
    dO = _dO(240, B, H, T, dv, "bf16")
    d = {n: dev(x[n]) for n in NAMES}
    log("backward T4096: GPU")
    out = rd.rodimus_scan_backward(d["q"], d["k"], d["v"], d["g"], d["theta"], dev(dO))
    torch.cuda.synchronize()
    for kk in GRADS:
        assert torch.isfinite(out[kk]).all(), kk
    heads = [(0, 0), (3, 15)]
    log(f"backward T4096: oracle on (b,h) {heads}")
    for b, h in heads:
        sub = [x[n].values[b:b + 1, h:h + 1].astype(np.float64) for n in NAMES]
        ref = oracle.scan_backward(*sub, dO.values[b:b + 1, h:h + 1].astype(np.float64))
        ref["dtau"] = ref.pop("dtheta")
        got = {kk: out[kk][b:b + 1, h:h + 1] for kk in GRADS}
        _check(got, ref, TOL["bf16"], f"T4096 (b,h)=({b},{h})")
