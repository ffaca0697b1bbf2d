"""GPU parity of rodimus_decode_step against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, err, host, log

pytestmark = pytest.mark.gpu


def _run_steps(sets, S_dev, steps, in_place=True):
    outs = []
    for s in range(steps):
        x = sets[s % len(sets)]
        d = {n: dev(x[n]) for n in ("q", "k", "v", "g", "theta")}
        if in_place:
            o = rd.rodimus_decode_step(d["q"], d["k"], d["v"], d["g"], d["theta"], S_dev)
        else:
            S_new = torch.empty_like(S_dev)
            o = rd.rodimus_decode_step(d["q"], d["k"], d["v"], d["g"], d["theta"], S_dev, S_new)
            S_dev = S_new
        outs.append(o)
    return outs, S_dev


def _oracle_steps(sets, S, steps):
    outs = []
    for s in range(steps):
        x = sets[s % len(sets)]
        o, S = oracle.decode(x["q"].f64(), x["k"].f64(), x["v"].f64(), x["g"].f64(),
                             x["theta"].f64(), S)
        outs.append(o)
    return outs, S


@pytest.mark.parametrize("dtype,N,H,dk,dv,steps", [
    ("bf16", 256, 16, 128, 128, 8),   # the decode batch workload, 8 steps of its input pool
    ("bf16", 3, 2, 64, 64, 5),
    ("fp32", 4, 3, 128, 128, 5),
    ("fp32", 2, 2, 16, 32, 6),
    ("fp32", 2, 3, 48, 80, 4),        # generic kernel (not a power of two)
    ("bf16", 5, 1, 128, 64, 3),
    ("bf16", 1, 1, 32, 64, 3),
])
def test_decode_parity(dtype, N, H, dk, dv, steps):
    log(f"decode parity {dtype} N={N} H={H} dk={dk} dv={dv} steps={steps}")
    sets = workloads.decode_pool(4, N, H, dk, dv, pool=8, dtype=dtype)
    rng = np.random.default_rng(99)
    S0 = (0.1 * rng.standard_normal((N, H, dk, dv))).astype(np.float32)
    S_dev = torch.from_numpy(S0.copy()).cuda()
    outs, S_dev = _run_steps(sets, S_dev, steps)
    torch.cuda.synchronize()
    ref_outs, S_ref = _oracle_steps(sets, S0.astype(np.float64), steps)
    for o, r in zip(outs, ref_outs):
        assert err(host(o), r) <= TOL[dtype]
    e = err(host(S_dev), S_ref)
    log(f"  state err {e:.3e}")
    assert e <= 1e-4


def test_decode_in_place_equals_out_of_place():
    sets = workloads.decode_pool(4, 8, 4, 128, 128, pool=2)
    S0 = torch.randn(8, 4, 128, 128, device="cuda", dtype=torch.float32, generator=None) * 0.1
    o1, S1 = _run_steps(sets, S0.clone(), 3, in_place=True)
    o2, S2 = _run_steps(sets, S0.clone(), 3, in_place=False)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    for a, b in zip(o1, o2):
        assert torch.equal(a, b)


def test_decode_reduces_to_linear_attention_update():
    """tau = -inf: S' = S + k^T v exactly as in plain linear attention."""
    N, H, dk, dv = 2, 2, 128, 128
    x = workloads.decode_pool(4, N, H, dk, dv, pool=1, dtype="fp32")[0]
    d = {n: dev(x[n]) for n in ("q", "k", "v", "g")}
    tau = torch.full_like(d["g"], float("-inf"))
    S = torch.zeros(N, H, dk, dv, device="cuda")
    o = rd.rodimus_decode_step(d["q"], d["k"], d["v"], d["g"], tau, S)
    torch.cuda.synchronize()
    k, v, q = x["k"].f64(), x["v"].f64(), x["q"].f64()
    Sref = k[..., :, None] * v[..., None, :]
    assert err(host(S), Sref) < 1e-6
    assert err(host(o), np.einsum("nhi,nhij->nhj", q, Sref)) < 1e-5


def test_decode_zero_sizes():
    q = torch.empty(0, 16, 128, device="cuda", dtype=torch.bfloat16)
    S = torch.empty(0, 16, 128, 128, device="cuda")
    o = rd.rodimus_decode_step(q, q, q, q, q, S)
    assert o.shape == (0, 16, 128)


def test_decode_large_in_place_state_streamed_loads():
    """An in-place state larger than 640 MiB (N = 704: 738 MB) is read with
    streaming loads, a smaller one with ordinary loads: both against the
    oracle on sampled (n, h) pairs, and the large one bitwise equal to the same
    steps written out of place."""
    N, H, d, steps = 704, 16, 128, 3
    log(f"decode N={N} in place ({N * H * d * d * 4 / 1e6:.0f} MB state)")
    sets = workloads.decode_pool(44, N, H, d, d, pool=steps)
    S = workloads.device_normal((N, H, d, d), 45).float() * 0.1
    S_start = host(S)
    S2 = S.clone()
    outs_in, outs_out = [], []
    for s in range(steps):
        x = {n: dev(sets[s][n]) for n in ("q", "k", "v", "g", "theta")}
        outs_in.append(rd.rodimus_decode_step(x["q"], x["k"], x["v"], x["g"], x["theta"], S))
        S_new = torch.empty_like(S2)
        outs_out.append(rd.rodimus_decode_step(x["q"], x["k"], x["v"], x["g"], x["theta"], S2, S_new))
        S2 = S_new
    torch.cuda.synchronize()
    assert torch.equal(S, S2)
    for a, b in zip(outs_in, outs_out):
        assert torch.equal(a, b)
    pairs = [(0, 0), (351, 7), (703, 15), (511, 3)]
    ns, hs = [p[0] for p in pairs], [p[1] for p in pairs]
    Sr = S_start[ns, hs][:, None]
    for s in range(steps):
        sub = [sets[s][n].values[ns, hs][:, None].astype(np.float64) for n in ("q", "k", "v", "g", "theta")]
        ro, Sr = oracle.decode(*sub, Sr)
        assert err(host(outs_in[s][ns, hs])[:, None], ro) <= TOL["bf16"]
    e = err(host(S[ns, hs])[:, None], Sr)
    log(f"  state err on sampled pairs {e:.2e}")
    assert e <= 1e-4
