"""GPU parity of rodimus_scan_prefill_varlen (packed ragged batches).

Each sequence of a packed batch is checked against the oracle's scan of that
sequence alone (with its own S0), on both paths: matrix cores (bf16,
dk = dv = 128, held to the bf16 bar) and the generic fp32 path (1e-4).  A
packed batch of equal lengths must equal the batched call bit for bit (same
plan, same kernels).  Cases include empty and one-token sequences, lengths
around the 32/64-token boundaries, and a long sequence beside a short one so
that the segment plan gives the short one empty segments."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, err, host, log

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "theta")


def _packed(seed, H, lengths, dk, dv, dtype, with_state=True):
    total = int(np.sum(lengths))
    x = workloads.packed_scan_inputs(seed, H, total, dk, dv, dtype)
    cu = workloads.cu_seqlens(lengths)
    S0 = (np.random.default_rng(seed + 1).standard_normal((len(lengths), H, dk, dv)) * 0.5).astype(np.float32) \
        if with_state else None
    return x, cu, S0


def _run(x, cu, S0, max_seqlen, chunk=64):
    d = {n: dev(x[n]) for n in NAMES}
    cud = torch.from_numpy(cu).cuda()
    S0d = None if S0 is None else torch.from_numpy(S0).cuda()
    o, ST = rd.rodimus_scan_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["theta"], cud, max_seqlen, S0d,
                                           chunk)
    torch.cuda.synchronize()
    return host(o), host(ST)


def _check_each(x, cu, S0, o, ST, tol, label):
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        sub = [x[n].values[None, :, a:b].astype(np.float64) for n in NAMES]
        s0 = None if S0 is None else S0[s:s + 1].astype(np.float64)
        ro, rST = oracle.scan(*sub, s0)
        es = err(ST[s:s + 1], rST)
        eo = err(o[None, :, a:b], ro) if b > a else 0.0
        worst = max(worst, eo, es)
        assert eo <= tol and es <= tol, (label, s, b - a, eo, es)
    log(f"  {label}: {len(cu) - 1} sequences, worst err {worst:.2e}")


@pytest.mark.parametrize("lengths", [
    [0, 1, 33, 64, 150, 300, 7],
    [31, 32, 63, 65, 128, 129],
])
def test_varlen_matrix_core_matches_the_oracle_per_sequence(lengths):
    H = 2
    x, cu, S0 = _packed(300 + len(lengths), H, lengths, 128, 128, "bf16")
    o, ST = _run(x, cu, S0, max(lengths))
    _check_each(x, cu, S0, o, ST, TOL["bf16"], f"mfma {lengths}")


def test_varlen_long_beside_short_uses_empty_segments():
    # two (b,h) pairs per sequence: the plan cuts the 5000-token sequence into
    # many segments; the 17-token one has tokens in the first only
    lengths = [5000, 17]
    x, cu, S0 = _packed(310, 2, lengths, 128, 128, "bf16")
    o, ST = _run(x, cu, S0, 5000)
    _check_each(x, cu, S0, o, ST, TOL["bf16"], "long + short")


def test_varlen_generic_fp32():
    lengths = [5, 0, 70, 33]
    x, cu, S0 = _packed(320, 3, lengths, 32, 48, "fp32")
    o, ST = _run(x, cu, S0, 70, chunk=32)
    _check_each(x, cu, S0, o, ST, 1e-4, "fp32 dk32 dv48")


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("bf16", 128, 32), ("fp32", 64, 16)])
def test_varlen_equal_lengths_equal_the_batched_call(dtype, d, chunk):
    B, H, T = 3, 2, 200
    x = workloads.scan_inputs(330, B, H, T, d, d, dtype)
    S0 = torch.from_numpy((np.random.default_rng(331).standard_normal((B, H, d, d)) * 0.5).astype(np.float32)).cuda()
    db = {n: dev(x[n]) for n in NAMES}
    ob, STb = rd.rodimus_scan_prefill(db["q"], db["k"], db["v"], db["g"], db["theta"], S0, chunk)
    # the same sequences packed per head: [H, B*T, d]
    dp = {n: t.permute(1, 0, 2, 3).reshape(H, B * T, d).contiguous() for n, t in db.items()}
    cu = torch.tensor([0, T, 2 * T, 3 * T], dtype=torch.int32, device="cuda")
    op, STp = rd.rodimus_scan_prefill_varlen(dp["q"], dp["k"], dp["v"], dp["g"], dp["theta"], cu, T, S0, chunk)
    torch.cuda.synchronize()
    assert torch.equal(op, ob.permute(1, 0, 2, 3).reshape(H, B * T, d))
    assert torch.equal(STp, STb)


def test_varlen_dynamic_batch_workload_sampled():
    c = workloads.CONFIGS["prefill_varlen_N64_16K"]
    L = workloads.ragged_lengths(c["seed"], c["N"], c["total"], c["min_len"])
    x = workloads.packed_scan_inputs(c["seed"], c["H"], c["total"], c["dk"], c["dv"], c["dtype"])
    cu = workloads.cu_seqlens(L)
    d = {n: dev(x[n]) for n in NAMES}
    o, ST = rd.rodimus_scan_prefill_varlen(d["q"], d["k"], d["v"], d["g"], d["theta"], torch.from_numpy(cu).cuda(),
                                           int(L.max()), None, c["chunk"])
    torch.cuda.synchronize()
    o, ST = host(o), host(ST)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    for s in (0, int(np.argmax(L)), c["N"] - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in (0, c["H"] - 1):
            sub = [x[n].values[None, h:h + 1, a:b].astype(np.float64) for n in NAMES]
            ro, rST = oracle.scan(*sub)
            eo, es = err(o[None, h:h + 1, a:b], ro), err(ST[s:s + 1, h:h + 1], rST)
            log(f"  dynamic batch seq {s} (len {b - a}) head {h}: o {eo:.2e} S_T {es:.2e}")
            assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_varlen_malformed_offsets_stay_in_bounds():
    # a decreasing offset and one past the end: the spans are clamped on the
    # device, so the call completes and writes nothing past the output tensor
    H, total, d = 2, 100, 128
    x = workloads.packed_scan_inputs(340, H, total, d, d, "bf16")
    dd = {n: dev(x[n]) for n in NAMES}
    buf = torch.zeros((H * total + 64, d), dtype=torch.bfloat16, device="cuda")
    buf[H * total:] = 7.0                       # guard rows after the output
    o = buf[:H * total].view(H, total, d)
    cu = torch.tensor([0, 50, 30, 200], dtype=torch.int32, device="cuda")
    rd.rodimus_scan_prefill_varlen(dd["q"], dd["k"], dd["v"], dd["g"], dd["theta"], cu, 100, None, 64, o=o)
    torch.cuda.synchronize()
    assert torch.all(buf[H * total:] == 7.0)


@pytest.mark.parametrize("N", [4096, 5000])
def test_varlen_many_short_sequences(N):
    # N = 4096: the largest batch ranked by length; N = 5000: ordered by chunk count
    rng = np.random.default_rng(350 + N)
    lengths = rng.integers(0, 10, size=N)
    lengths[N // 2] = 200                       # one long request in the middle
    x, cu, S0 = _packed(351, 1, lengths, 128, 128, "bf16")
    o, ST = _run(x, cu, S0, int(lengths.max()))
    picks = sorted({0, 1, N // 2, N - 1, *rng.integers(0, N, size=40).tolist()})
    for s in picks:
        a, b = int(cu[s]), int(cu[s + 1])
        sub = [x[n].values[None, :, a:b].astype(np.float64) for n in NAMES]
        ro, rST = oracle.scan(*sub, S0[s:s + 1].astype(np.float64))
        es = err(ST[s:s + 1], rST)
        eo = err(o[None, :, a:b], ro) if b > a else 0.0
        assert eo <= TOL["bf16"] and es <= TOL["bf16"], (N, s, b - a, eo, es)
    log(f"  {N} sequences: {len(picks)} checked")


@pytest.mark.parametrize("N", [3000, 5000, 20000])
def test_varlen_order_in_workspace(N):
    """The longest-first order the packed prefill writes into its workspace
    after the plan's own bytes: ranked by length, ties by index, up to 4096
    sequences; counted by 64-token chunk count beyond (equal counts in any
    order).  Either way a permutation of the sequences."""
    rng = np.random.default_rng(360 + N)
    lengths = rng.integers(0, 300, size=N)
    lengths[N // 3] = 2000                      # one long request
    lengths[rng.integers(0, N, size=20)] = 0    # and some empty ones
    H, d = 1, 128
    x, cu, _ = _packed(361, H, lengths, d, d, "bf16", with_state=False)
    maxlen = int(lengths.max())
    base = rd.rodimus_scan_prefill_workspace_bytes(N, H, maxlen, d, d, 64, rd.BF16)
    need = rd.rodimus_scan_prefill_varlen_workspace_bytes(N, H, maxlen, d, d, 64, rd.BF16)
    assert need - base >= 4 * N
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    dd = {n: dev(x[n]) for n in NAMES}
    rd.rodimus_scan_prefill_varlen(dd["q"], dd["k"], dd["v"], dd["g"], dd["theta"], torch.from_numpy(cu).cuda(),
                                   maxlen, None, 64, workspace=ws, want_state=False)
    torch.cuda.synchronize()
    order = ws[base:base + 4 * N].view(torch.int32).cpu().numpy()
    assert np.array_equal(np.sort(order), np.arange(N))
    if N <= 4096:
        assert np.array_equal(order, np.lexsort((np.arange(N), -lengths)))
    else:
        key = np.minimum((lengths + 63) // 64, 4095)[order]
        assert np.all(key[:-1] >= key[1:])
    log(f"  {N} sequences: order checked")

