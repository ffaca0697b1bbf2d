"""GPU parity at the full workload sizes, in the launch configuration the bench
times, element by element against the fp64 oracle.

* 1.6B-shaped prefill (B4 T4096 H16 d128): every output and final state.
* Long-context prefill (B1 T131072 H16 d128): every head over the whole length.
* Decode (256 sequences x 16 heads, 1000 in-place steps): every (n,h) pair's
  output at steps 0, 1 and 7 and its state after step 7; 64 seeded pairs
  (corners included) at steps across the 1000 and their final state.
* SW-SKA (B1 T32768 H16 d128, w4096): the first and last query row of every
  32-query block of every head -- every wave of the launch computes two of the
  checked rows, whatever the block-to-workgroup order -- plus the rows around
  the window edge (t = 4095, 4096, 4097) of every head.

Each check logs, besides the bar (max|x-r|/max|r|), the worst (b,h) slice and
the element-wise error with a 1e-3 max|r| floor."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, errs, fmt, host, log

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "theta")
ORACLE_THREADS = 16


def check(name, x, r, bar, unit_axes=2, per_unit_bar=None):
    e = errs(x, r, unit_axes)
    log(fmt(name, e))
    assert e["err"] <= bar, (name, e)
    if per_unit_bar is not None:
        assert e["per_unit"] <= per_unit_bar, (name, e)
    return e


def test_prefill_1p6b_T4096_full_parity():
    c = workloads.CONFIGS["prefill_1p6b_T4096"]
    log("prefill_1p6b_T4096: generating inputs")
    x = workloads.scan_inputs(c["seed"], c["B"], c["H"], c["T"], c["dk"], c["dv"], c["dtype"])
    d = {n: dev(x[n]) for n in NAMES}
    log("prefill_1p6b_T4096: GPU")
    o, ST = rd.rodimus_scan_prefill(*(d[n] for n in NAMES), None, c["chunk"])
    torch.cuda.synchronize()
    log("prefill_1p6b_T4096: oracle")
    ro, rST = oracle.scan(*(x[n].f64() for n in NAMES), nthreads=ORACLE_THREADS)
    check("o", host(o), ro, TOL["bf16"], per_unit_bar=TOL["bf16"])
    check("S_T", host(ST), rST, TOL["bf16"], per_unit_bar=TOL["bf16"])


def test_prefill_long_T131072_full_parity():
    c = workloads.CONFIGS["prefill_long_T131072"]
    log("prefill_long_T131072: generating inputs")
    x = workloads.scan_inputs(c["seed"], c["B"], c["H"], c["T"], c["dk"], c["dv"], c["dtype"],
                              gate_mu=c["gate_mu"])
    d = {n: dev(x[n]) for n in NAMES}
    log("prefill_long_T131072: GPU")
    o, ST = rd.rodimus_scan_prefill(*(d[n] for n in NAMES), None, c["chunk"])
    torch.cuda.synchronize()
    del d
    oh, STh = host(o), host(ST)
    del o, ST
    log(f"prefill_long_T131072: oracle on all {c['H']} heads")
    args = [x[n].values.astype(np.float64) for n in NAMES]
    del x
    ro, rST = oracle.scan(*args, nthreads=ORACLE_THREADS)
    del args
    check("o", oh, ro, TOL["bf16"], per_unit_bar=TOL["bf16"])
    check("S_T", STh, rST, TOL["bf16"], per_unit_bar=TOL["bf16"])
    # the last 4096 positions, where the state has carried 127K tokens
    check("o[-4096:]", oh[:, :, -4096:], ro[:, :, -4096:], TOL["bf16"])
    # the first position of every 8192-token segment-plan boundary region
    seg_starts = np.arange(0, c["T"], 8192)
    check("o[segment starts]", oh[:, :, seg_starts], ro[:, :, seg_starts], TOL["bf16"])


def test_decode_N256_all_pairs_and_1000_steps():
    c = workloads.CONFIGS["decode_N256"]
    N, H, dk, dv, steps = c["N"], c["H"], c["dk"], c["dv"], c["steps"]
    sets = workloads.decode_pool(c["seed"], N, H, dk, dv, pool=c["pool"], dtype=c["dtype"])
    dsets = [{n: dev(s[n]) for n in NAMES} for s in sets]
    S = torch.zeros(N, H, dk, dv, device="cuda")
    full_steps = (0, 1, 7)
    rng = np.random.default_rng(4004)
    flat = np.concatenate([[0, H - 1, (N - 1) * H, N * H - 1],
                           rng.choice(np.arange(1, N * H - 1), size=60, replace=False)])
    ns, hs = flat // H, flat % H
    keep = {0, 1, 7, 8, 63, 64, 127, 128, 255, 256, 499, 500, 511, 512, 997, 998, 999}
    full_o, sample_o = {}, {}
    S7 = None
    log("decode_N256: 1000 in-place steps on the GPU")
    for s in range(steps):
        o = rd.rodimus_decode_step(*(dsets[s % len(dsets)][n] for n in NAMES), S)
        if s in full_steps:
            full_o[s] = host(o)
        if s in keep:
            sample_o[s] = host(o[ns, hs])
        if s == 7:
            S7 = host(S)
    torch.cuda.synchronize()
    S_end = host(S)
    assert np.all(np.isfinite(S_end))

    log("decode_N256: oracle on all 4096 (n,h) pairs, steps 0..7")
    Sref = np.zeros((N, H, dk, dv))
    for s in range(8):
        xs = sets[s % len(sets)]
        ro, Sref = oracle.decode(*(xs[n].f64() for n in NAMES), Sref)
        if s in full_steps:
            check(f"o step {s}", full_o[s], ro, TOL["bf16"], per_unit_bar=TOL["bf16"])
    check("S after step 7", S7, Sref, 1e-4, per_unit_bar=1e-4)
    del Sref

    log(f"decode_N256: oracle on {flat.size} (n,h) pairs over {steps} steps")
    Sp = np.zeros((flat.size, 1, dk, dv))
    worst = 0.0
    for s in range(steps):
        xs = sets[s % len(sets)]
        sub = [xs[n].values[ns, hs][:, None].astype(np.float64) for n in NAMES]
        ro, Sp = oracle.decode(*sub, Sp)
        if s in keep:
            e = errs(sample_o[s][:, None], ro)
            worst = max(worst, e["err"])
            assert e["err"] <= TOL["bf16"] and e["per_unit"] <= TOL["bf16"], (s, e)
    log(f"  sampled outputs: worst err over the kept steps {worst:.3e}")
    check("S after 1000 steps (sampled pairs)", S_end[ns, hs][:, None], Sp, 1e-4, per_unit_bar=1e-4)


def test_swska_T32768_w4096_every_wave():
    c = workloads.CONFIGS["swska_T32768_w4096"]
    B, H, T, D, w = c["B"], c["H"], c["T"], c["dk"], c["window"]
    log("swska_T32768_w4096: inputs")
    x = workloads.swska_inputs(c["seed"], B, H, T, D, D)
    d = {n: dev(x[n]) for n in ("q", "k", "v")}
    log("swska_T32768_w4096: GPU")
    o = rd.sw_ska_attn(d["q"], d["k"], d["v"], w)
    torch.cuda.synchronize()
    o = host(o)
    assert np.all(np.isfinite(o))
    starts = np.arange(0, T, 32)
    ts = np.unique(np.concatenate([starts, starts + 31, [w - 1, w, w + 1]]))
    rows = (np.arange(H)[:, None] * T + ts[None, :]).reshape(-1)
    log(f"swska_T32768_w4096: oracle on {rows.size} rows ({ts.size} per head)")
    r = oracle.swska(x["q"].f64(), x["k"].f64(), x["v"].f64(), w, rows=rows, nthreads=ORACLE_THREADS)
    got = o.reshape(-1, D)[rows].reshape(H, ts.size, D)
    ref = r.reshape(-1, D)[rows].reshape(H, ts.size, D)
    check("o (rows per head)", got, ref, TOL["bf16"], unit_axes=1, per_unit_bar=TOL["bf16"])
    check("o (per row)", got.reshape(-1, D), ref.reshape(-1, D), TOL["bf16"], unit_axes=1)
    edge = np.searchsorted(ts, [w - 1, w, w + 1])
    check("o (window edge rows)", got[:, edge], ref[:, edge], TOL["bf16"], unit_axes=1)
