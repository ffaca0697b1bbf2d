"""GPU parity of rodimus_scan_backward_varlen (the backward over a packed
ragged batch).

Every sequence of a packed batch is checked against the oracle's backward of
that sequence alone (with its own S0 and dS_T), on both paths: matrix cores
(bf16, dk = dv = 128, held to the bf16 bar) and the generic fp32 path (1e-4).
A packed batch of equal lengths must equal the batched backward bit for bit.
Cases: empty and one-token sequences, lengths around the 32/64-token
boundaries, a long sequence beside a short one (the short one then has empty
checkpoint segments, through which dS_T must pass unchanged), fast decays that
send some halves to the exact fallback, the dynamic-batch workload on sampled
sequences, and a malformed offset table (nothing written outside the
gradients)."""
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


def _packed(seed, H, lengths, dk, dv, dtype):
    total = int(np.sum(lengths))
    x = workloads.packed_scan_inputs(seed, H, total, dk, dv, dtype)
    rng = np.random.default_rng(seed + 1)
    dO = workloads.Tensor(workloads.round_to(rng.standard_normal((H, total, dv)), dtype), dtype)
    N = len(lengths)
    S0 = (rng.standard_normal((N, H, dk, dv)) * 0.5).astype(np.float32)
    dST = (rng.standard_normal((N, H, dk, dv)) * 0.5).astype(np.float32)
    return x, dO, workloads.cu_seqlens(lengths), S0, dST


def _run(x, dO, cu, S0, dST, max_seqlen):
    d = {n: dev(x[n]) for n in NAMES}
    out = rd.rodimus_scan_backward_varlen(d["q"], d["k"], d["v"], d["g"], d["theta"], dev(dO),
                                          torch.from_numpy(cu).cuda(), max_seqlen,
                                          torch.from_numpy(S0).cuda(), torch.from_numpy(dST).cuda())
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def _check_each(x, dO, cu, S0, dST, out, tol, label):
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:  # nothing but the final-state gradient reaches S0
            assert np.array_equal(out["dS0"][s], dST[s].astype(np.float64)), (label, s)
            continue
        sub = [x[n].values[None, :, a:b].astype(np.float64) for n in NAMES]
        ref = oracle.scan_backward(*sub, dO.values[None, :, a:b].astype(np.float64),
                                   S0[s:s + 1].astype(np.float64), dST[s:s + 1].astype(np.float64), nthreads=8)
        ref["dtau"] = ref.pop("dtheta")
        errs = {k: err(out[k][None, :, a:b], ref[k]) for k in GRADS}
        errs["dS0"] = err(out["dS0"][s:s + 1], ref["dS0"])
        worst = max(worst, max(errs.values()))
        for k, e in errs.items():
            assert e <= tol, (label, s, b - a, k, e)
    log(f"  {label}: {len(cu) - 1} sequences, worst err {worst:.2e}")


@pytest.mark.parametrize("lengths", [
    [0, 1, 33, 64, 150, 300, 7],
    [31, 32, 63, 65, 128, 129],
])
def test_varlen_backward_matrix_core_matches_the_oracle_per_sequence(lengths):
    H = 2
    x, dO, cu, S0, dST = _packed(400 + len(lengths), H, lengths, 128, 128, "bf16")
    out = _run(x, dO, cu, S0, dST, max(lengths))
    _check_each(x, dO, cu, S0, dST, out, TOL["bf16"], f"mfma {lengths}")


def test_varlen_backward_long_beside_short_uses_empty_segments():
    # 4 (b,h) pairs: the plan cuts the 5000-token sequence into 64 checkpoint
    # segments; the 17-token one has tokens in the first only, and its dS_T
    # reaches it through 63 empty segments
    lengths = [5000, 17]
    x, dO, cu, S0, dST = _packed(410, 2, lengths, 128, 128, "bf16")
    out = _run(x, dO, cu, S0, dST, 5000)
    _check_each(x, dO, cu, S0, dST, out, TOL["bf16"], "long + short")


def test_varlen_backward_generic_fp32():
    lengths = [5, 0, 70, 33]
    x, dO, cu, S0, dST = _packed(420, 3, lengths, 32, 48, "fp32")
    out = _run(x, dO, cu, S0, dST, 70)
    _check_each(x, dO, cu, S0, dST, out, 1e-4, "fp32 dk32 dv48")


def test_varlen_backward_fast_decay_fallback():
    # gate logits ~ -10 with tau ~ +3 over part of the middle sequence: log2 a ~
    # -14 per token, so those halves take the exact fallback routine
    lengths = [90, 200, 45]
    x, dO, cu, S0, dST = _packed(430, 2, lengths, 128, 128, "bf16")
    lo, hi = int(cu[1]) + 70, int(cu[1]) + 110
    x["g"].values[:, lo:hi] = workloads.round_to(x["g"].values[:, lo:hi] - 10.0, "bf16")
    x["theta"].values[:, lo:hi] = workloads.round_to(np.abs(x["theta"].values[:, lo:hi]) + 3.0, "bf16")
    out = _run(x, dO, cu, S0, dST, 200)
    _check_each(x, dO, cu, S0, dST, out, TOL["bf16"], "fallback")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_varlen_backward_equal_lengths_equal_the_batched_call(dtype, d):
    B, H, T = 3, 2, 200
    x = workloads.scan_inputs(440, B, H, T, d, d, dtype)
    rng = np.random.default_rng(441)
    dO = workloads.Tensor(workloads.round_to(rng.standard_normal((B, H, T, d)), dtype), dtype)
    S0 = torch.from_numpy((rng.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)).cuda()
    dST = torch.from_numpy((rng.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)).cuda()
    db = {n: dev(x[n]) for n in NAMES}
    dOb = dev(dO)
    ob = rd.rodimus_scan_backward(db["q"], db["k"], db["v"], db["g"], db["theta"], dOb, S0, dST)
    # the same sequences packed per head: [H, B*T, d]
    pk = lambda t: t.permute(1, 0, 2, 3).reshape(H, B * T, d).contiguous()
    dp = {n: pk(t) for n, t in db.items()}
    cu = torch.tensor([0, T, 2 * T, 3 * T], dtype=torch.int32, device="cuda")
    op = rd.rodimus_scan_backward_varlen(dp["q"], dp["k"], dp["v"], dp["g"], dp["theta"], pk(dOb), cu, T, S0, dST)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(op[k], pk(ob[k])), k
    assert torch.equal(op["dS0"], ob["dS0"])


def test_varlen_backward_dynamic_batch_workload_sampled():
    c = workloads.CONFIGS["prefill_varlen_N64_16K"]
    L = workloads.ragged_lengths(c["seed"], c["N"], c["total"], c["min_len"])
    x = workloads.packed_scan_inputs(c["seed"], c["H"], c["total"], c["dk"], c["dv"], c["dtype"])
    rng = np.random.default_rng(c["seed"] + 50)
    dO = workloads.Tensor(workloads.round_to(rng.standard_normal((c["H"], c["total"], c["dv"])), "bf16"), "bf16")
    cu = workloads.cu_seqlens(L)
    d = {n: dev(x[n]) for n in NAMES}
    out = rd.rodimus_scan_backward_varlen(d["q"], d["k"], d["v"], d["g"], d["theta"], dev(dO),
                                          torch.from_numpy(cu).cuda(), int(L.max()))
    torch.cuda.synchronize()
    out = {k: host(v) for k, v in out.items()}
    for k in GRADS + ("dS0",):
        assert np.all(np.isfinite(out[k])), k
    for s in (0, int(np.argmax(L)), c["N"] - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in (0, c["H"] - 1):
            sub = [x[n].values[None, h:h + 1, a:b].astype(np.float64) for n in NAMES]
            ref = oracle.scan_backward(*sub, dO.values[None, h:h + 1, a:b].astype(np.float64), nthreads=8)
            ref["dtau"] = ref.pop("dtheta")
            errs = {k: err(out[k][None, h:h + 1, a:b], ref[k]) for k in GRADS}
            errs["dS0"] = err(out["dS0"][s:s + 1, h:h + 1], ref["dS0"])
            log(f"  dynamic batch seq {s} (len {b - a}) head {h}: "
                + " ".join(f"{k} {e:.2e}" for k, e in errs.items()))
            for k, e in errs.items():
                assert e <= TOL["bf16"], (s, h, k, e)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 32)])
def test_varlen_backward_malformed_offsets_stay_in_bounds(dtype, d):
    # a decreasing offset and one past the end: the spans are clamped on the
    # device, so the call completes and writes nothing past the gradients
    H, total = 2, 100
    x = workloads.packed_scan_inputs(450, H, total, d, d, dtype)
    rng = np.random.default_rng(451)
    dO = workloads.Tensor(workloads.round_to(rng.standard_normal((H, total, d)), dtype), dtype)
    dd = {n: dev(x[n]) for n in NAMES}
    bufs, out = {}, {}
    for k in GRADS:
        bufs[k] = torch.zeros((H * total + 64, d), dtype=torch.float32, device="cuda")
        bufs[k][H * total:] = 7.0               # guard rows after the gradient
        out[k] = bufs[k][:H * total].view(H, total, d)
    cu = torch.tensor([0, 50, 30, 200], dtype=torch.int32, device="cuda")
    rd.rodimus_scan_backward_varlen(dd["q"], dd["k"], dd["v"], dd["g"], dd["theta"], dev(dO), cu, 100, out=out)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.all(bufs[k][H * total:] == 7.0), k


@pytest.mark.parametrize("N", [4096, 5000])
def test_varlen_backward_many_short_sequences(N):
    # N = 4096: the largest batch ranked by length; N = 5000: ordered by chunk count
    rng = np.random.default_rng(460 + N)
    lengths = rng.integers(0, 10, size=N)
    lengths[N // 3] = 150
    x, dO, cu, S0, dST = _packed(461, 1, lengths, 128, 128, "bf16")
    out = _run(x, dO, cu, S0, dST, int(lengths.max()))
    picks = sorted({0, N // 3, N - 1, *rng.integers(0, N, size=30).tolist()})
    for s in picks:
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            assert np.array_equal(out["dS0"][s], dST[s].astype(np.float64)), (N, s)
            continue
        sub = [x[n].values[None, :, a:b].astype(np.float64) for n in NAMES]
        ref = oracle.scan_backward(*sub, dO.values[None, :, a:b].astype(np.float64),
                                   S0[s:s + 1].astype(np.float64), dST[s:s + 1].astype(np.float64))
        ref["dtau"] = ref.pop("dtheta")
        for k in GRADS:
            e = err(out[k][None, :, a:b], ref[k])
            assert e <= TOL["bf16"], (N, s, k, e)
        assert err(out["dS0"][s:s + 1], ref["dS0"]) <= TOL["bf16"], (N, s)
    log(f"  {N} sequences: {len(picks)} checked")
