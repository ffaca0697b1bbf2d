"""GPU parity of sw_ska_decode_step (one SW-SKA token per sequence over
ring-buffer window caches) against the oracle's dense softmax per row: the
decode output for a token at position t is row t of SW-SKA over the
sequence, so the oracle is oracle.swska on the sequence (or on the window's
keys gathered from the caches in position order)."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, err, host, log

pytestmark = pytest.mark.gpu


def _empty_caches(N, H, W, d):
    kc = torch.zeros(N, W, d, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(N, H, W, d, dtype=torch.bfloat16, device="cuda")
    return kc, vc


@pytest.mark.parametrize("d", [128, 64])
def test_steps_from_empty_cache_match_rows(d):
    N, H, T, W = 3, 5, 230, 96          # the window wraps twice; H not a multiple of 16
    log(f"swska decode: {T} steps from an empty cache, d={d}, W={W}")
    x = workloads.swska_inputs(31 + d, N, H, T, d, d)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    kc, vc = _empty_caches(N, H, W, d)
    pos = torch.zeros(N, dtype=torch.int32, device="cuda")
    outs = []
    for t in range(T):
        outs.append(rd.sw_ska_decode_step(q[:, :, t].contiguous(), k[:, t].contiguous(),
                                          v[:, :, t].contiguous(), kc, vc, pos).clone())
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2)
    ref = oracle.swska(x["q"].f64(), x["k"].f64(), x["v"].f64(), W)
    e = err(host(o), ref)
    log(f"  err o {e:.3e}")
    assert e <= TOL["bf16"]
    # the positions advanced, and slot p mod W holds position p for the last W positions
    assert torch.equal(pos.cpu(), torch.full((N,), T, dtype=torch.int32))
    for p in range(T - W, T):
        assert torch.equal(kc[:, p % W], k[:, p])
        assert torch.equal(vc[:, :, p % W], v[:, :, p])
    # and the decode rows agree with the prefill kernel on the same sequence
    op = rd.sw_ska_attn(q, k, v, W)
    assert err(host(o), host(op)) <= TOL["bf16"]


def _gather_window(kc_n, vc_n, t, W):
    """Keys [L, d] and values [H, L, d] of positions max(0, t-W+1) .. t, in order,
    read from one sequence's ring-buffer caches (host arrays)."""
    ps = list(range(max(0, t - W + 1), t + 1))
    slots = [p % W for p in ps]
    return kc_n[slots], vc_n[:, slots]


@pytest.mark.parametrize("W", [1, 64, 300])
def test_ragged_positions_against_window_oracle(W):
    N, H, d = 6, 4, 128
    ts = [0, 1, W - 1, W, W + 7, 1000]
    log(f"swska decode: ragged positions {ts}, W={W}")
    rng = np.random.default_rng(40 + W)
    kc = torch.from_numpy(workloads.round_to(rng.standard_normal((N, W, d)), "bf16")).cuda().to(torch.bfloat16)
    vc = torch.from_numpy(workloads.round_to(rng.standard_normal((N, H, W, d)), "bf16")).cuda().to(torch.bfloat16)
    x = workloads.swska_inputs(50 + W, N, H, 1, d, d)
    qn, kn, vn = dev(x["q"])[:, :, 0].contiguous(), dev(x["k"])[:, 0].contiguous(), dev(x["v"])[:, :, 0].contiguous()
    pos = torch.tensor(ts, dtype=torch.int32, device="cuda")
    o = rd.sw_ska_decode_step(qn, kn, vn, kc, vc, pos)
    torch.cuda.synchronize()
    assert torch.equal(pos.cpu(), torch.tensor(ts, dtype=torch.int32) + 1)
    kch, vch = host(kc), host(vc)
    for n, t in enumerate(ts):
        kw, vw = _gather_window(kch[n], vch[n], t, W)
        L = kw.shape[0]
        qs = np.zeros((1, H, L, d))
        qs[0, :, -1] = host(qn[n])
        ref = oracle.swska(qs, kw[None], vw[None], W, rows=[h * L + L - 1 for h in range(H)])
        e = err(host(o[n]), ref[0, :, -1])
        assert e <= TOL["bf16"], (n, t, e)


def test_window_one_returns_v_new():
    N, H, d = 4, 3, 64
    x = workloads.swska_inputs(61, N, H, 1, d, d)
    qn, kn, vn = dev(x["q"])[:, :, 0].contiguous(), dev(x["k"])[:, 0].contiguous(), dev(x["v"])[:, :, 0].contiguous()
    kc, vc = _empty_caches(N, H, 1, d)
    pos = torch.tensor([0, 5, 9, 100], dtype=torch.int32, device="cuda")
    o = rd.sw_ska_decode_step(qn, kn, vn, kc, vc, pos)
    torch.cuda.synchronize()
    assert torch.equal(o, vn)


def test_zero_sizes_are_noops():
    d = 128
    z = torch.empty(0, 3, d, dtype=torch.bfloat16, device="cuda")
    o = rd.sw_ska_decode_step(z, torch.empty(0, d, dtype=torch.bfloat16, device="cuda"), z,
                              torch.empty(0, 16, d, dtype=torch.bfloat16, device="cuda"),
                              torch.empty(0, 3, 16, d, dtype=torch.bfloat16, device="cuda"),
                              torch.empty(0, dtype=torch.int32, device="cuda"))
    assert o.shape == (0, 3, d)


def test_decode_N64_w4096_sampled_heads():
    N, H, d, W, t = 64, 16, 128, 4096, 5000
    log("swska decode N64 w4096: caches on the device")
    kc = workloads.device_normal((N, W, d), 91)
    vc = workloads.device_normal((N, H, W, d), 92)
    x = workloads.swska_inputs(93, N, H, 1, d, d)
    qn, kn, vn = dev(x["q"])[:, :, 0].contiguous(), dev(x["k"])[:, 0].contiguous(), dev(x["v"])[:, :, 0].contiguous()
    pos = torch.full((N,), t, dtype=torch.int32, device="cuda")
    o = rd.sw_ska_decode_step(qn, kn, vn, kc, vc, pos)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    for n in (0, 17, 63):
        kw, vw = _gather_window(host(kc[n]), host(vc[n]), t, W)
        qs = np.zeros((1, H, W, d))
        qs[0, :, -1] = host(qn[n])
        ref = oracle.swska(qs, kw[None], vw[None], W, rows=[h * W + W - 1 for h in range(H)], nthreads=8)
        e = err(host(o[n]), ref[0, :, -1])
        log(f"  n={n}: err o {e:.3e}")
        assert e <= TOL["bf16"]


@pytest.mark.parametrize("N,H,W,d", [(128, 8, 4100, 128), (512, 1, 4096, 128), (256, 8, 4100, 64),
                                     (512, 1, 4096, 64)])
def test_long_splits_against_window_oracle(N, H, W, d):
    # enough (sequence, split, head group) workgroups for the 1024-slot splits
    # (two heads per workgroup at H = 8, one at H = 1), at both head sizes;
    # W = 4100 leaves a ragged last split; positions from an empty window to
    # several wraps
    log(f"swska decode long splits: N={N} H={H} W={W} d={d}")
    kc = workloads.device_normal((N, W, d), 71 + H + d)
    vc = workloads.device_normal((N, H, W, d), 72 + H + d)
    x = workloads.swska_inputs(73 + H + d, N, H, 1, d, d)
    qn, kn, vn = dev(x["q"])[:, :, 0].contiguous(), dev(x["k"])[:, 0].contiguous(), dev(x["v"])[:, :, 0].contiguous()
    rng = np.random.default_rng(74 + H)
    ts = rng.integers(0, 3 * W, size=N)
    ts[:6] = [0, 1, 1023, 1024, W - 1, 2 * W + 5]
    pos = torch.from_numpy(ts.astype(np.int32)).cuda()
    o = rd.sw_ska_decode_step(qn, kn, vn, kc, vc, pos)
    torch.cuda.synchronize()
    assert torch.equal(pos.cpu(), torch.from_numpy(ts.astype(np.int32) + 1))
    for n in sorted({0, 1, 2, 3, 4, 5, N // 2, N - 1}):
        t = int(ts[n])
        ps = np.arange(max(0, t - W + 1), t + 1)
        slots = torch.from_numpy(ps % W).cuda()
        kw, vw = host(kc[n].index_select(0, slots)), host(vc[n].index_select(1, slots))
        L = len(ps)
        qs = np.zeros((1, H, L, d))
        qs[0, :, -1] = host(qn[n])
        ref = oracle.swska(qs, kw[None], vw[None], W, rows=[h * L + L - 1 for h in range(H)], nthreads=8)
        e = err(host(o[n]), ref[0, :, -1])
        assert e <= TOL["bf16"], (n, t, e)
