"""The decode entry points inside HIP graphs.  Both launch kernels only (no
allocation, no memset) on the caller's stream, so a serving loop can capture
several steps once and replay them.  Each test captures a few steps, replays
the graph several times with eager work and synchronisations in between, and
checks every replay against the same steps run eagerly."""
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
