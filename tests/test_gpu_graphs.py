"""The entry points inside HIP graphs.  They launch kernels only (no
allocation, no memset) on the caller's stream, with scratch only in the
caller's workspace, so a serving or training loop can capture them once and
replay them: several decode steps, and one prefill (segment states, combine,
output pass) or one backward (state passes, combine, gradients, fallback list
and its counter).  Each test replays the graph several times with eager work
and synchronisations in between, and checks every replay bit for bit against
the same calls run eagerly; the decode graphs are also checked against the
fp64 oracle, replay after replay (the replays continue the same sequences).
The last test captures a two-layer chain of both decode mixers (Rodimus then
SW-SKA in each layer, each mixer's output feeding the next one's queries) over
several steps into one graph and checks every output and state against the
oracle's chain."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, err, host, log

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
    S_ref = np.zeros((N, H, dk, dv))
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        steps(S_eager, eager_outs)        # eager work between replays
        torch.cuda.synchronize()
        log(f"replay {rep}")
        assert torch.equal(S_graph, S_eager), rep
        for i in range(K):
            assert torch.equal(outs[i], eager_outs[i]), (rep, i)
            ro, S_ref = oracle.decode(*(sets[i][n].f64() for n in NAMES), S_ref)
            e = err(host(outs[i]), ro)
            assert e <= TOL["bf16"], (rep, i, e)
        es = err(host(S_graph), S_ref)
        log(f"  against the oracle after {K * (rep + 1)} steps: S err {es:.2e}")
        assert es <= 1e-4, rep


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
        kc_before, vc_before, pos_before = host(kc_g), host(vc_g), pos_g.cpu().numpy().copy()
        graph.replay()
        torch.cuda.synchronize()
        steps(kc_e, vc_e, pos_e, eager_outs, ws_e)
        torch.cuda.synchronize()
        log(f"replay {rep}")
        assert torch.equal(pos_g, pos_e), rep
        assert torch.equal(kc_g, kc_e) and torch.equal(vc_g, vc_e), rep
        for i in range(K):
            assert torch.equal(outs[i], eager_outs[i]), (rep, i)
        # against the oracle: each step's output is the SW-SKA row of its
        # position over the window of keys/values the caches held, with the
        # replay's own tokens appended in order
        ref = _swska_decode_oracle(kc_before, vc_before, pos_before, toks, W)
        e = err(np.stack([host(o) for o in outs]), ref)
        log(f"  against the oracle: err {e:.2e}")
        assert e <= TOL["bf16"], rep


def _swska_decode_oracle(kc, vc, pos, toks, W):
    """fp64 outputs of len(toks) SW-SKA decode steps from caches kc [N,W,d],
    vc [N,H,W,d] (host copies) at positions pos [N]: step i appends token i at
    position pos+i (slot (pos+i) mod W) and attends over the last W positions."""
    kc, vc = kc.copy(), vc.copy()
    N, H, d = vc.shape[0], vc.shape[1], vc.shape[3]
    outs = np.zeros((len(toks), N, H, d))
    for i, (qn, kn, vn) in enumerate(toks):
        qh, kh, vh = host(qn), host(kn), host(vn)
        for n in range(N):
            t = int(pos[n]) + i
            kc[n, t % W] = kh[n]
            vc[n, :, t % W] = vh[n]
            ps = list(range(max(0, t - W + 1), t + 1))
            sl = [p % W for p in ps]
            L = len(ps)
            qs = np.zeros((1, H, L, d))
            qs[0, :, -1] = qh[n]
            r = oracle.swska(qs, kc[n][sl][None], vc[n][:, sl][None], W, rows=[h * L + L - 1 for h in range(H)])
            outs[i, n] = r[0, :, -1]
    return outs


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


def test_two_layer_mixer_chain_decode_graph_against_oracle():
    """Rodimus+ decode, two layers: per layer a Rodimus decode step (global
    recurrent mixer) then an SW-SKA decode step (local window mixer), all
    steps of a few tokens captured into one graph.  The projections and the
    residual stream between mixers are outside this library; in their place
    each mixer's bf16 output is the next mixer's query (layer l's SW-SKA query
    is its Rodimus output, layer l+1's Rodimus query is layer l's SW-SKA
    output), so the graph's launches depend on one another in order.  Every
    output, state and cache is checked against the oracle's chain, which
    rounds each intermediate output to bf16 itself."""
    N, H, d, W, K, L = 4, 4, 128, 48, 5, 2
    rx = [workloads.decode_pool(200 + l, N, H, d, d, pool=K) for l in range(L)]   # k, v, g, theta per step
    q0 = workloads.decode_pool(210, N, H, d, d, pool=K)                           # layer 0's queries
    sx = [workloads.swska_inputs(220 + l, N, H, K, d, d) for l in range(L)]      # k_new, v_new per step
    r_in = [[{n: dev(rx[l][i][n]) for n in ("k", "v", "g", "theta")} for i in range(K)] for l in range(L)]
    q_in = [dev(q0[i]["q"]) for i in range(K)]
    s_in = [[(dev(sx[l]["k"])[:, i].contiguous(), dev(sx[l]["v"])[:, :, i].contiguous()) for i in range(K)]
            for l in range(L)]

    def fresh_state():
        return dict(S=[torch.zeros(N, H, d, d, device="cuda") for _ in range(L)],
                    kc=[torch.zeros(N, W, d, dtype=torch.bfloat16, device="cuda") for _ in range(L)],
                    vc=[torch.zeros(N, H, W, d, dtype=torch.bfloat16, device="cuda") for _ in range(L)],
                    pos=[torch.zeros(N, dtype=torch.int32, device="cuda") for _ in range(L)],
                    ws=[torch.empty(rd.sw_ska_decode_workspace_bytes(N, H, d, d, W), dtype=torch.uint8,
                                    device="cuda") for _ in range(L)],
                    o_r=[[torch.empty(N, H, d, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
                         for _ in range(L)],
                    o_s=[[torch.empty(N, H, d, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
                         for _ in range(L)])

    def run(st):
        for i in range(K):
            q = q_in[i]
            for l in range(L):
                x = r_in[l][i]
                rd.rodimus_decode_step(q, x["k"], x["v"], x["g"], x["theta"], st["S"][l], o=st["o_r"][l][i])
                kn, vn = s_in[l][i]
                rd.sw_ska_decode_step(st["o_r"][l][i], kn, vn, st["kc"][l], st["vc"][l], st["pos"][l],
                                      o=st["o_s"][l][i], workspace=st["ws"][l])
                q = st["o_s"][l][i]

    gg = fresh_state()
    graph, _ = _capture(lambda: run(gg))   # the warm-up before capture advances gg; reset below

    S_ref = [np.zeros((N, H, d, d)) for _ in range(L)]
    K_hist = [np.zeros((N, 0, d)) for _ in range(L)]
    V_hist = [np.zeros((N, H, 0, d)) for _ in range(L)]
    e_st = fresh_state()
    for rep in range(3):
        for l in range(L):
            gg["S"][l].zero_(); gg["kc"][l].zero_(); gg["vc"][l].zero_(); gg["pos"][l].zero_()
        graph.replay()
        torch.cuda.synchronize()
        if rep == 0:
            run(e_st)                      # eager work between replays, same chain
            torch.cuda.synchronize()
            for l in range(L):
                assert torch.equal(e_st["S"][l], gg["S"][l])
                for i in range(K):
                    assert torch.equal(e_st["o_r"][l][i], gg["o_r"][l][i])
                    assert torch.equal(e_st["o_s"][l][i], gg["o_s"][l][i])
            # the oracle's chain over the same K steps
            worst = 0.0
            for i in range(K):
                q = q0[i]["q"].f64()
                for l in range(L):
                    x = rx[l][i]
                    o_r, S_ref[l] = oracle.decode(q, *(x[n].f64() for n in ("k", "v", "g", "theta")), S_ref[l])
                    o_r_bf = workloads.round_to(o_r, "bf16").astype(np.float64)
                    K_hist[l] = np.concatenate([K_hist[l], sx[l]["k"].f64()[:, i:i + 1]], axis=1)
                    V_hist[l] = np.concatenate([V_hist[l], sx[l]["v"].f64()[:, :, i:i + 1]], axis=2)
                    T = i + 1
                    qs = np.zeros((N, H, T, d))
                    qs[:, :, -1] = o_r_bf
                    rows = [(n * H + h) * T + T - 1 for n in range(N) for h in range(H)]
                    o_s = oracle.swska(qs, K_hist[l], V_hist[l], W, rows=rows)[:, :, -1]
                    e1 = err(host(gg["o_r"][l][i]), o_r)
                    e2 = err(host(gg["o_s"][l][i]), o_s)
                    worst = max(worst, e1, e2)
                    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"], (i, l, e1, e2)
                    q = workloads.round_to(o_s, "bf16").astype(np.float64)
            for l in range(L):
                es = err(host(gg["S"][l]), S_ref[l])
                assert es <= 1e-4, (l, es)
                assert torch.equal(gg["pos"][l].cpu(), torch.full((N,), K, dtype=torch.int32))
            log(f"two-layer chain: worst output err {worst:.2e} against the oracle")
            ref_o = [[host(gg["o_r"][l][i]) for i in range(K)] for l in range(L)]
            ref_s = [[host(gg["o_s"][l][i]) for i in range(K)] for l in range(L)]
        else:
            # replays from the same zero state repeat the first replay bit for bit
            for l in range(L):
                for i in range(K):
                    assert np.array_equal(host(gg["o_r"][l][i]), ref_o[l][i]), (rep, l, i)
                    assert np.array_equal(host(gg["o_s"][l][i]), ref_s[l][i]), (rep, l, i)
            log(f"two-layer chain: replay {rep} repeats replay 0")
