"""The entry points inside HIP graphs.  They launch kernels only (no
allocation, no memset) on the caller's stream, with scratch only in the
caller's workspace, so a serving or training loop can capture them once and
replay them: several decode steps, and one prefill (segment states, combine,
output pass) or one backward (state passes, combine, gradients, fallback list
and its counter).  Each test replays the graph several times with eager work
and synchronisations in between, and checks every replay bit for bit against
the same calls run eagerly."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import workloads
from tests.gpu_helpers import dev, log

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "theta")


def test_rodimus_decode_steps_replayed_from_a_graph():
    N, H, dk, dv, K = 8, 4, 128, 128, 6
    sets = workloads.decode_pool(101, N, H, dk, dv, pool=K)
    dsets = [{n: dev(s[n]) for n in NAMES} for s in sets]
    S_graph = torch.zeros(N, H, dk, dv, device="cuda")
    outs = [torch.empty(N, H, dv, dtype=torch.bfloat16, device="cuda") for _ in range(K)]

    def steps(S, os_):
        for i in range(K):
            rd.rodimus_decode_step(*(dsets[i][n] for n in NAMES), S, o=os_[i])

    # warm up on a side stream (as torch requires before capture), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps(torch.zeros_like(S_graph), [torch.empty_like(o) for o in outs])
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(S_graph, outs)

    S_eager = torch.zeros_like(S_graph)
    S_graph.zero_()
    eager_outs = [torch.empty_like(o) for o in outs]
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        steps(S_eager, eager_outs)        # eager work between replays
        torch.cuda.synchronize()
        log(f"replay {rep}")
        assert torch.equal(S_graph, S_eager), rep
        for i in range(K):
            assert torch.equal(outs[i], eager_outs[i]), (rep, i)


def test_swska_decode_steps_replayed_from_a_graph():
    N, H, d, W, K = 4, 3, 128, 96, 5
    x = workloads.swska_inputs(102, N, H, K, d, d)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    toks = [(q[:, :, i].contiguous(), k[:, i].contiguous(), v[:, :, i].contiguous()) for i in range(K)]
    ws_g = torch.empty(rd.sw_ska_decode_workspace_bytes(N, H, d, d, W), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws_g)

    def caches():
        c = workloads.device_normal((N, W, d), 103), workloads.device_normal((N, H, W, d), 104)
        return c[0], c[1], torch.tensor([0, 5, W - 1, 3 * W + 7], dtype=torch.int32, device="cuda")

    kc_g, vc_g, pos_g = caches()
    outs = [torch.empty(N, H, d, dtype=torch.bfloat16, device="cuda") for _ in range(K)]

    def steps(kc, vc, pos, os_, ws):
        for i in range(K):
            rd.sw_ska_decode_step(*toks[i], kc, vc, pos, o=os_[i], workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kw, vw, pw = caches()
        steps(kw, vw, pw, [torch.empty_like(o) for o in outs], ws_g)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(kc_g, vc_g, pos_g, outs, ws_g)

    # the replays keep appending tokens; the eager side does the same steps
    kc_g.copy_(caches()[0]); vc_g.copy_(caches()[1]); pos_g.copy_(caches()[2])
    kc_e, vc_e, pos_e = caches()
    eager_outs = [torch.empty_like(o) for o in outs]
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        steps(kc_e, vc_e, pos_e, eager_outs, ws_e)
        torch.cuda.synchronize()
        log(f"replay {rep}")
        assert torch.equal(pos_g, pos_e), rep
        assert torch.equal(kc_g, kc_e) and torch.equal(vc_g, vc_e), rep
        for i in range(K):
            assert torch.equal(outs[i], eager_outs[i]), (rep, i)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up, as torch requires before capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    return graph, out


def test_prefill_replayed_from_a_graph():
    # B*H = 16: 16 segments, so the call is all three kernels
    B, H, T, d = 2, 8, 1000, 128
    x = workloads.scan_inputs(105, B, H, T, d, d, "bf16")
    dd = {n: dev(x[n]) for n in NAMES}
    S0 = workloads.device_normal((B, H, d, d), 106).float() * 0.5
    need = rd.rodimus_scan_prefill_workspace_bytes(B, H, T, d, d, 64)
    ws_g = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_g = torch.empty(B, H, T, d, dtype=torch.bfloat16, device="cuda")
    ST_g = torch.empty(B, H, d, d, device="cuda")

    graph, _ = _capture(lambda: rd.rodimus_scan_prefill(*(dd[n] for n in NAMES), S0, 64, o=o_g, S_T=ST_g,
                                                        workspace=ws_g))
    ws_e = torch.empty_like(ws_g)
    for rep in range(3):
        o_g.zero_(); ST_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        o_e, ST_e = rd.rodimus_scan_prefill(*(dd[n] for n in NAMES), S0, 64, workspace=ws_e)
        torch.cuda.synchronize()
        log(f"prefill replay {rep}")
        assert torch.equal(o_g, o_e) and torch.equal(ST_g, ST_e), rep


def test_backward_replayed_from_a_graph():
    # 11 checkpoint segments per (b,h); a stretch of fast decay sends some
    # halves to the fallback list, whose counter the state pass resets
    B, H, T, d = 1, 4, 700, 128
    x = workloads.scan_inputs(107, B, H, T, d, d, "bf16")
    x["g"].values[:, :, 300:340] = workloads.round_to(x["g"].values[:, :, 300:340] - 10.0, "bf16")
    x["theta"].values[:, :, 300:340] = workloads.round_to(np.abs(x["theta"].values[:, :, 300:340]) + 3.0, "bf16")
    dd = {n: dev(x[n]) for n in NAMES}
    dO = workloads.device_normal((B, H, T, d), 108)
    S0 = workloads.device_normal((B, H, d, d), 109).float() * 0.5
    dST = workloads.device_normal((B, H, d, d), 110).float() * 0.5
    ws_g = torch.empty(rd.rodimus_scan_backward_workspace_bytes(B, H, T, d, d), dtype=torch.uint8, device="cuda")
    graph, out_g = _capture(lambda: rd.rodimus_scan_backward(*(dd[n] for n in NAMES), dO, S0, dST, workspace=ws_g))
    ws_e = torch.empty_like(ws_g)
    for rep in range(3):
        for t in out_g.values():
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        out_e = rd.rodimus_scan_backward(*(dd[n] for n in NAMES), dO, S0, dST, workspace=ws_e)
        torch.cuda.synchronize()
        log(f"backward replay {rep}")
        for k in out_e:
            assert torch.equal(out_g[k], out_e[k]), (rep, k)
