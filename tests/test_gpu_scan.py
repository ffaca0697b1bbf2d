"""GPU parity of rodimus_scan_prefill against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, err, host, log

pytestmark = pytest.mark.gpu


def run_gpu(x, chunk, S0=None):
    d = {n: dev(x[n]) for n in ("q", "k", "v", "g", "theta")}
    S0d = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).cuda()
    o, ST = rd.rodimus_scan_prefill(d["q"], d["k"], d["v"], d["g"], d["theta"], S0d, chunk)
    torch.cuda.synchronize()
    return host(o), host(ST)


def run_oracle(x, S0=None, heads=None):
    arrs = [x[n].f64() for n in ("q", "k", "v", "g", "theta")]
    return oracle.scan(*arrs, S0=None if S0 is None else np.asarray(S0, np.float64), nthreads=8)


def check(x, chunk, dtype, S0=None, tol=None):
    o, ST = run_gpu(x, chunk, S0)
    ro, rST = run_oracle(x, S0)
    eo, es = err(o, ro), err(ST, rST)
    log(f"  err o {eo:.3e}  S_T {es:.3e}")
    t = TOL[dtype] if tol is None else tol
    assert eo <= t and es <= t
    return o, ST


def test_tiny_fp32_workload():
    """B=1, H=2, T=256, dk=16, dv=32, fp32, C=32, gate logits N(0,1), S0 = 0."""
    c = workloads.CONFIGS["tiny_fp32_scan"]
    log("scan tiny_fp32_scan")
    x = workloads.scan_inputs(c["seed"], c["B"], c["H"], c["T"], c["dk"], c["dv"], "fp32")
    check(x, c["chunk"], "fp32")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dtype,B,H,T,dk,dv", [
    ("fp32", 1, 2, 200, 16, 32),
    ("fp32", 2, 1, 131, 64, 48),
    ("bf16", 2, 2, 300, 128, 128),
    ("bf16", 1, 3, 77, 48, 80),
])
def test_scan_shapes_and_chunks(chunk, dtype, B, H, T, dk, dv):
    log(f"scan {dtype} B={B} H={H} T={T} dk={dk} dv={dv} C={chunk}")
    x = workloads.scan_inputs(11, B, H, T, dk, dv, dtype)
    check(x, chunk, dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_scan_with_initial_state(dtype):
    B, H, T, dk, dv = 2, 2, 150, 128, 128
    x = workloads.scan_inputs(12, B, H, T, dk, dv, dtype)
    S0 = np.random.default_rng(5).standard_normal((B, H, dk, dv)).astype(np.float32)
    log(f"scan S0 {dtype}")
    check(x, 64, dtype, S0=S0)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 129])
def test_scan_ragged_lengths(T):
    x = workloads.scan_inputs(13, 1, 2, T, 128, 128, "bf16")
    log(f"scan ragged T={T}")
    check(x, 64, "bf16")


def test_scan_empty_sequence_copies_state():
    B, H, dk, dv = 2, 3, 128, 128
    q = torch.empty(B, H, 0, dk, device="cuda", dtype=torch.bfloat16)
    S0 = torch.randn(B, H, dk, dv, device="cuda")
    o, ST = rd.rodimus_scan_prefill(q, q, q, q, q, S0, 64)
    torch.cuda.synchronize()
    assert o.shape == (B, H, 0, dv) and torch.equal(ST, S0)
    o, ST = rd.rodimus_scan_prefill(q, q, q, q, q, None, 64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ST) == 0


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_scan_extreme_gates(dtype):
    """Mixed-sign extreme logits: decay spans far beyond the factorised range."""
    B, H, T, dk, dv = 1, 2, 160, 128, 128
    x = workloads.scan_inputs(14, B, H, T, dk, dv, dtype)
    rng = np.random.default_rng(3)
    x["g"] = workloads.Tensor(workloads.round_to(rng.choice([-8.0, 8.0], size=x["g"].shape), dtype), dtype)
    x["theta"] = workloads.Tensor(workloads.round_to(rng.choice([-2.0, 4.0], size=x["g"].shape), dtype), dtype)
    log(f"scan extreme gates {dtype}")
    check(x, 64, dtype)


def test_scan_reset_gates():
    B, H, T, dk, dv = 1, 2, 96, 128, 128
    x = workloads.scan_inputs(15, B, H, T, dk, dv, "fp32")
    x["g"] = workloads.Tensor(np.full(x["g"].shape, -40.0, np.float32), "fp32")
    x["theta"] = workloads.Tensor(np.full(x["g"].shape, 40.0, np.float32), "fp32")
    log("scan reset gates")
    check(x, 32, "fp32")


@pytest.mark.parametrize("chunk", [64, 32])
def test_scan_fast_decay_within_a_half(chunk):
    """g ~ N(-2, 0.5), theta ~ N(2, 0.5): about 2.7 log2 units of decay per token,
    so a 64-token chunk spans ~2^173 (beyond the factorised range) while each
    32-token half spans ~2^86 (within it); a stretch of much stronger decay
    (g ~ -8, about 10 log2 units per token) puts some halves beyond it, into
    the token-by-token branch."""
    B, H, T, dk, dv = 1, 3, 900, 128, 128
    x = workloads.scan_inputs(17, B, H, T, dk, dv, "bf16")
    rng = np.random.default_rng(9)
    g = -2 + 0.5 * rng.standard_normal(x["g"].shape)
    g[:, :, 500:560] -= 6.0
    x["g"] = workloads.Tensor(workloads.round_to(g, "bf16"), "bf16")
    x["theta"] = workloads.Tensor(workloads.round_to(2 + 0.5 * rng.standard_normal(x["g"].shape), "bf16"), "bf16")
    log(f"scan fast decay C={chunk}")
    check(x, chunk, "bf16")


@pytest.mark.parametrize("chunk", [64, 32])
def test_scan_decay_just_past_the_factorised_range(chunk):
    """g ~ N(-3, 0.5), theta ~ N(3, 0.5): about 4.2 log2 units of decay per
    token, ~2^134 per 32-token half, just past the factorised range (Kh would
    reach 2^134): every chunk takes the token-by-token branch."""
    B, H, T, dk, dv = 1, 2, 700, 128, 128
    x = workloads.scan_inputs(18, B, H, T, dk, dv, "bf16")
    rng = np.random.default_rng(10)
    x["g"] = workloads.Tensor(workloads.round_to(-3 + 0.5 * rng.standard_normal(x["g"].shape), "bf16"), "bf16")
    x["theta"] = workloads.Tensor(workloads.round_to(3 + 0.5 * rng.standard_normal(x["g"].shape), "bf16"), "bf16")
    log(f"scan decay just past the factorised range C={chunk}")
    check(x, chunk, "bf16")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_scan_slow_decay(dtype):
    """g ~ N(4,1), theta ~ N(-2,1): a ~ 0.998, long-range carry across chunks."""
    B, H, T, dk, dv = 1, 2, 700, 128, 128
    x = workloads.scan_inputs(16, B, H, T, dk, dv, dtype)
    rng = np.random.default_rng(8)
    x["g"] = workloads.Tensor(workloads.round_to(4 + rng.standard_normal(x["g"].shape), dtype), dtype)
    x["theta"] = workloads.Tensor(workloads.round_to(-2 + rng.standard_normal(x["g"].shape), dtype), dtype)
    log(f"scan slow decay {dtype}")
    check(x, 64, dtype)


def test_scan_linear_attention_reduction():
    """tau = -inf: a = beta = 1; compare with causal linear attention."""
    B, H, T, dk, dv = 1, 2, 130, 128, 128
    x = workloads.scan_inputs(17, B, H, T, dk, dv, "fp32")
    x["theta"] = workloads.Tensor(np.full(x["g"].shape, -np.inf, np.float32), "fp32")
    o, ST = run_gpu(x, 64)
    q, k, v = x["q"].f64(), x["k"].f64(), x["v"].f64()
    KV = np.cumsum(k[..., :, None] * v[..., None, :], axis=2)
    ref = np.einsum("bhti,bhtij->bhtj", q, KV)
    assert err(o, ref) <= 1e-4 and err(ST, KV[:, :, -1]) <= 1e-4


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_scan_split_resume_and_decode_equivalence(dtype):
    B, H, T, dk, dv, T1 = 1, 2, 200, 128, 128, 75
    x = workloads.scan_inputs(18, B, H, T, dk, dv, dtype)
    d = {n: dev(x[n]) for n in ("q", "k", "v", "g", "theta")}
    o, ST = rd.rodimus_scan_prefill(d["q"], d["k"], d["v"], d["g"], d["theta"], None, 64)
    a = {n: t[:, :, :T1].contiguous() for n, t in d.items()}
    b = {n: t[:, :, T1:].contiguous() for n, t in d.items()}
    oa, Sa = rd.rodimus_scan_prefill(a["q"], a["k"], a["v"], a["g"], a["theta"], None, 64)
    ob, Sb = rd.rodimus_scan_prefill(b["q"], b["k"], b["v"], b["g"], b["theta"], Sa, 64)
    # decode: T steps from zero
    S = torch.zeros(B, H, dk, dv, device="cuda")
    od = [rd.rodimus_decode_step(*(d[n][:, :, t].contiguous() for n in ("q", "k", "v", "g", "theta")), S)
          for t in range(T)]
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert err(host(torch.cat([oa, ob], dim=2)), host(o)) <= tol
    assert err(host(Sb), host(ST)) <= tol
    assert err(host(torch.stack(od, dim=2)), host(o)) <= tol
    assert err(host(S), host(ST)) <= tol


def test_scan_deterministic():
    x = workloads.scan_inputs(19, 2, 4, 333, 128, 128, "bf16")
    o1, s1 = run_gpu(x, 64)
    o2, s2 = run_gpu(x, 64)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
