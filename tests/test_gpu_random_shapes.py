"""Seeded random-shape sweep of every entry point against the oracle.

The cases are drawn from fixed seeds: batch and head counts, lengths, head
sizes, chunk sizes, dtypes, gate means, initial states, windows, scales and
cache positions in combinations that the hand-picked cases of the other files
do not list (half of the scan cases take the matrix-core path, bf16 with
dk = dv = 128; the rest the generic path).  Each case is held to the same bar
as the rest: err = max|x - r| / max|r| per output tensor, 2e-2 for bf16 inputs
and 1e-4 for fp32."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, err, host, log

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "theta")
GRADS = ("dq", "dk", "dv", "dg", "dtau")
DIMS = [16, 32, 48, 64, 80, 96, 112, 128]


def _scan_cases(n, seed, tmax):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        mfma = i % 2 == 0
        dtype = "bf16" if mfma or rng.random() < 0.5 else "fp32"
        dk, dv = (128, 128) if mfma else (int(rng.choice(DIMS)), int(rng.choice(DIMS)))
        cases.append(dict(seed=seed * 100 + i, dtype=dtype, B=int(rng.integers(1, 3)),
                          H=int(rng.integers(1, 4)), T=int(rng.integers(1, tmax)), dk=dk, dv=dv,
                          chunk=int(rng.choice([16, 32, 64])), S0=bool(rng.random() < 0.5),
                          dST=bool(rng.random() < 0.5), gate_mu=float(rng.choice([0.0, 0.5, 3.0]))))
    return cases


def _scan_id(c):
    return f"{c['dtype']}-B{c['B']}H{c['H']}T{c['T']}-{c['dk']}x{c['dv']}-C{c['chunk']}-mu{c['gate_mu']}"


def _state(rng, c, on):
    return (rng.standard_normal((c["B"], c["H"], c["dk"], c["dv"])) * 0.5).astype(np.float32) if on else None


def _cuda(a):
    return None if a is None else torch.from_numpy(a).cuda()


def _f64(a):
    return None if a is None else a.astype(np.float64)


@pytest.mark.parametrize("c", _scan_cases(40, 71, 700), ids=_scan_id)
def test_prefill_random_shape(c):
    log(f"prefill {_scan_id(c)} S0={c['S0']}")
    x = workloads.scan_inputs(c["seed"], c["B"], c["H"], c["T"], c["dk"], c["dv"], c["dtype"], gate_mu=c["gate_mu"])
    S0 = _state(np.random.default_rng(c["seed"] + 1), c, c["S0"])
    d = {n: dev(x[n]) for n in NAMES}
    o, ST = rd.rodimus_scan_prefill(*(d[n] for n in NAMES), _cuda(S0), c["chunk"])
    torch.cuda.synchronize()
    ro, rST = oracle.scan(*(x[n].f64() for n in NAMES), S0=_f64(S0), nthreads=8)
    eo, es = err(host(o), ro), err(host(ST), rST)
    log(f"  err o {eo:.2e} S_T {es:.2e}")
    assert eo <= TOL[c["dtype"]] and es <= TOL[c["dtype"]]


def _lowrank_cases(n, seed, tmax):
    rng = np.random.default_rng(seed)
    return [dict(seed=seed * 100 + i, B=int(rng.integers(1, 4)), H=int(rng.integers(1, 20)),
                 T=int(rng.integers(1, tmax)), chunk=int(rng.choice([32, 64])), S0=bool(rng.random() < 0.5))
            for i in range(n)]


@pytest.mark.parametrize("c", _lowrank_cases(20, 77, 1500),
                         ids=lambda c: f"B{c['B']}H{c['H']}T{c['T']}-C{c['chunk']}-S0{int(c['S0'])}")
def test_prefill_lowrank_random_shape(c):
    """The low-rank prefill (bf16, d = 128, rank-16 gate factors) on random
    batch, head and length counts, which vary the segment plan: one segment,
    several with their states folded by the output pass, or many through the
    combine pass, and ragged last chunks."""
    names = ("q", "k", "v", "zg", "zt", "Ug", "bg", "Ut", "bt")
    log(f"prefill_lowrank B{c['B']} H{c['H']} T{c['T']} C{c['chunk']} S0={c['S0']}")
    x = workloads.lowrank_inputs(c["seed"], c["B"], c["H"], c["T"], 128, 128)
    S0 = _state(np.random.default_rng(c["seed"] + 1), dict(c, dk=128, dv=128), c["S0"])
    d = {n: dev(x[n]) for n in names}
    o, ST = rd.rodimus_scan_prefill_lowrank(*(d[n] for n in names), S0=_cuda(S0), chunk=c["chunk"])
    torch.cuda.synchronize()
    ro, rST = oracle.scan_lowrank(*(x[n].f64() for n in names), S0=_f64(S0), nthreads=8)
    eo, es = err(host(o), ro), err(host(ST), rST)
    log(f"  err o {eo:.2e} S_T {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("c", _scan_cases(24, 72, 400),
                         ids=lambda c: f"{c['dtype']}-B{c['B']}H{c['H']}T{c['T']}-{c['dk']}x{c['dv']}-mu{c['gate_mu']}")
def test_backward_random_shape(c):
    log(f"backward {c}")
    B, H, T, dv, dt = c["B"], c["H"], c["T"], c["dv"], c["dtype"]
    x = workloads.scan_inputs(c["seed"], B, H, T, c["dk"], dv, dt, gate_mu=c["gate_mu"])
    rng = np.random.default_rng(c["seed"] + 1)
    dO = workloads.Tensor(workloads.round_to(rng.standard_normal((B, H, T, dv)), dt), dt)
    S0, dST = _state(rng, c, c["S0"]), _state(rng, c, c["dST"])
    d = {n: dev(x[n]) for n in NAMES}
    out = rd.rodimus_scan_backward(*(d[n] for n in NAMES), dev(dO), _cuda(S0), _cuda(dST))
    torch.cuda.synchronize()
    ref = oracle.scan_backward(*(x[n].f64() for n in NAMES), dO.f64(), _f64(S0), _f64(dST), nthreads=8)
    ref["dtau"] = ref.pop("dtheta")
    errs = {k: err(host(out[k]), ref[k]) for k in GRADS + ("dS0",)}
    log("  " + " ".join(f"{k} {e:.2e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= TOL[dt], (k, e)


def _decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "bf16" if rng.random() < 0.6 else "fp32"
        d = 128 if i % 2 == 0 else None
        cases.append(dict(seed=seed * 100 + i, dtype=dtype, N=int(rng.integers(1, 40)), H=int(rng.integers(1, 6)),
                          dk=d or int(rng.choice(DIMS)), dv=d or int(rng.choice(DIMS)),
                          steps=int(rng.integers(1, 4)), out_of_place=bool(rng.random() < 0.5)))
    return cases


@pytest.mark.parametrize("c", _decode_cases(16, 73),
                         ids=lambda c: f"{c['dtype']}-N{c['N']}H{c['H']}-{c['dk']}x{c['dv']}-s{c['steps']}")
def test_decode_random_shape(c):
    log(f"decode {c}")
    N, H, dk, dv = c["N"], c["H"], c["dk"], c["dv"]
    sets = workloads.decode_pool(c["seed"], N, H, dk, dv, pool=c["steps"], dtype=c["dtype"])
    S = (np.random.default_rng(c["seed"] + 1).standard_normal((N, H, dk, dv)) * 0.5).astype(np.float32)
    Sd = torch.from_numpy(S).cuda()
    rS = S.astype(np.float64)
    for s in sets:
        dd = {n: dev(s[n]) for n in NAMES}
        Sout = torch.empty_like(Sd) if c["out_of_place"] else None
        o = rd.rodimus_decode_step(*(dd[n] for n in NAMES), Sd, Sout)
        if Sout is not None:
            Sd = Sout
        torch.cuda.synchronize()
        ro, rS = oracle.decode(*(s[n].f64() for n in NAMES), rS)
        eo = err(host(o), ro)
        assert eo <= TOL[c["dtype"]], eo
    es = err(host(Sd), rS)
    log(f"  err S {es:.2e}")
    assert es <= 1e-4


def _ska_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        T = int(rng.integers(1, 900))
        window = int(rng.choice([1, int(rng.integers(1, T + 1)), int(rng.integers(1, 2 * T + 2)), T + 300]))
        cases.append(dict(seed=seed * 100 + i, D=int(rng.choice([64, 128])), B=int(rng.integers(1, 3)),
                          H=int(rng.integers(1, 6)), T=T, window=window,
                          scale=None if rng.random() < 0.5 else float(rng.uniform(0.02, 0.3))))
    return cases


@pytest.mark.parametrize("c", _ska_cases(20, 74),
                         ids=lambda c: f"D{c['D']}-B{c['B']}H{c['H']}T{c['T']}-w{c['window']}")
def test_swska_random_shape(c):
    log(f"sw-ska {c}")
    x = workloads.swska_inputs(c["seed"], c["B"], c["H"], c["T"], c["D"], c["D"])
    o = rd.sw_ska_attn(dev(x["q"]), dev(x["k"]), dev(x["v"]), c["window"], c["scale"])
    torch.cuda.synchronize()
    ref = oracle.swska(x["q"].f64(), x["k"].f64(), x["v"].f64(), c["window"], scale=c["scale"], nthreads=8)
    e = err(host(o), ref)
    log(f"  err o {e:.2e}")
    assert e <= TOL["bf16"]


def _ska_decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        W = int(rng.choice([1, int(rng.integers(2, 256)), 256, 257, int(rng.integers(258, 1500))]))
        N = int(rng.integers(1, 8))
        cases.append(dict(seed=seed * 100 + i, D=int(rng.choice([64, 128])), N=N, H=int(rng.integers(1, 20)),
                          W=W, pos=[int(p) for p in rng.integers(0, 3 * W + 2, size=N)],
                          scale=None if rng.random() < 0.5 else float(rng.uniform(0.02, 0.3))))
    return cases


@pytest.mark.parametrize("c", _ska_decode_cases(20, 75),
                         ids=lambda c: f"D{c['D']}-N{c['N']}H{c['H']}-W{c['W']}")
def test_swska_decode_random_shape(c):
    log(f"sw-ska decode {c}")
    N, H, W, d = c["N"], c["H"], c["W"], c["D"]
    rng = np.random.default_rng(c["seed"])
    kc = torch.from_numpy(workloads.bf16_bits(rng.standard_normal((N, W, d))).view(np.int16)).cuda().view(torch.bfloat16)
    vc = torch.from_numpy(workloads.bf16_bits(rng.standard_normal((N, H, W, d))).view(np.int16)).cuda().view(torch.bfloat16)
    x = workloads.swska_inputs(c["seed"] + 1, N, H, 1, d, d)
    qn, kn, vn = dev(x["q"])[:, :, 0].contiguous(), dev(x["k"])[:, 0].contiguous(), dev(x["v"])[:, :, 0].contiguous()
    pos = torch.tensor(c["pos"], dtype=torch.int32, device="cuda")
    o = rd.sw_ska_decode_step(qn, kn, vn, kc, vc, pos, scale=c["scale"])
    torch.cuda.synchronize()
    assert pos.cpu().tolist() == [p + 1 for p in c["pos"]]
    kch, vch = host(kc), host(vc)
    for n, t in enumerate(c["pos"]):
        # the step wrote the new token into slot t mod W, so the caches now hold the whole window
        ps = list(range(max(0, t - W + 1), t + 1))
        kw, vw = kch[n][[p % W for p in ps]], vch[n][:, [p % W for p in ps]]
        L = len(ps)
        qs = np.zeros((1, H, L, d))
        qs[0, :, -1] = host(qn[n])
        ref = oracle.swska(qs, kw[None], vw[None], W, scale=c["scale"], rows=[h * L + L - 1 for h in range(H)])
        e = err(host(o[n]), ref[0, :, -1])
        assert e <= TOL["bf16"], (n, t, e)
        assert np.array_equal(kch[n][t % W], host(kn[n])) and np.array_equal(vch[n][:, t % W], host(vn[n]))
