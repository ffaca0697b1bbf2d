"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest

import gated_linear_attention_ddts_amd as rd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rodimus.h")

FAKE = 0x10000          # aligned, non-null; never dereferenced (validation fails first)
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_header_declares_the_exported_entry_points():
    assert declared_functions() == sorted(rd.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(rd.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for code in (rd.OK, rd.ERR_INVALID_ARG, rd.ERR_UNSUPPORTED, rd.ERR_HIP, rd.ERR_TOO_LARGE):
        s = rd.status_string(code)
        assert s.startswith("RODIMUS_")
    assert rd.status_string(12345) == "RODIMUS_UNKNOWN_STATUS"


def scan(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, tau=FAKE, S0=None, o=FAKE, S_T=None, B=1, H=1, T=8,
             dk=16, dv=16, chunk=64, dtype=rd.BF16, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return rd.lib().rodimus_scan_prefill(a["q"], a["k"], a["v"], a["g"], a["tau"], a["S0"], a["o"],
                                         a["S_T"], a["B"], a["H"], a["T"], a["dk"], a["dv"],
                                         a["chunk"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(g=None), dict(tau=None), dict(o=None),
    dict(q=MISALIGNED), dict(S0=MISALIGNED), dict(S_T=MISALIGNED),
    dict(B=-1), dict(H=-2), dict(T=-1), dict(dk=8), dict(dk=24), dict(dk=144), dict(dv=0),
    dict(dv=136), dict(chunk=8), dict(chunk=128), dict(chunk=-64), dict(dtype=2), dict(dtype=-1),
    dict(S0=FAKE, S_T=FAKE),
])
def test_scan_rejects(kw):
    assert scan(**kw) == rd.ERR_INVALID_ARG


def test_scan_empty_batch_is_noop():
    assert scan(B=0, q=None, k=None) == rd.OK
    assert scan(H=0, o=None) == rd.OK
    # T == 0 without S_T launches nothing
    assert scan(T=0, q=None, o=None) == rd.OK


def test_workspace_query():
    assert rd.rodimus_scan_prefill_workspace_bytes(1, 1, 8, 8, 16, 64, rd.BF16) == 0  # invalid dk
    n = rd.rodimus_scan_prefill_workspace_bytes(1, 16, 131072, 128, 128, 64, rd.BF16)
    assert n >= 0
    assert rd.rodimus_scan_prefill_workspace_bytes(4, 16, 4096, 128, 128, 0, rd.BF16) >= 0
    # empty problems need no workspace (and must not divide by zero)
    assert rd.rodimus_scan_prefill_workspace_bytes(2, 3, 0, 128, 128, 64, rd.BF16) == 0
    assert rd.rodimus_scan_prefill_workspace_bytes(0, 3, 100, 128, 128, 64, rd.BF16) == 0
    assert rd.rodimus_scan_prefill_workspace_bytes(1, 1, 1, 128, 128, 32, rd.BF16) == 0


def decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, tau=FAKE, S_in=FAKE, S_out=FAKE, o=FAKE, N=2, H=2,
             dk=16, dv=16, dtype=rd.BF16, stream=None)
    a.update(kw)
    return rd.lib().rodimus_decode_step(a["q"], a["k"], a["v"], a["g"], a["tau"], a["S_in"],
                                        a["S_out"], a["o"], a["N"], a["H"], a["dk"], a["dv"],
                                        a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(S_in=None), dict(S_out=None), dict(o=None), dict(v=MISALIGNED),
    dict(N=-1), dict(H=-1), dict(dk=0), dict(dv=20), dict(dtype=7),
    dict(S_out=FAKE + 16),  # partial overlap with S_in
])
def test_decode_rejects(kw):
    assert decode(**kw) == rd.ERR_INVALID_ARG


def test_decode_empty_is_noop():
    assert decode(N=0, q=None) == rd.OK


def ska(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=2, T=16, dk=128, dv=128, window=4,
             scale=0.088, dtype=rd.BF16, stream=None)
    a.update(kw)
    return rd.lib().sw_ska_attn(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["T"], a["dk"],
                                a["dv"], a["window"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(window=0), dict(window=-3), dict(scale=0.0), dict(scale=-1.0), dict(scale=float("inf")),
    dict(scale=float("nan")), dict(B=-1), dict(T=-5), dict(dk=7), dict(dtype=3),
])
def test_swska_rejects(kw):
    assert ska(**kw) == rd.ERR_INVALID_ARG


def test_swska_unsupported_shapes():
    assert ska(dk=128, dv=64) == rd.ERR_UNSUPPORTED
    assert ska(dk=32, dv=32) == rd.ERR_UNSUPPORTED
    assert ska(dtype=rd.F32) == rd.ERR_UNSUPPORTED
    # 32-bit byte offsets into k_shared and v: T * dk * 2 < 2^31
    assert ska(T=1 << 23) == rd.ERR_UNSUPPORTED
    assert ska(T=1 << 24, dk=64, dv=64) == rd.ERR_UNSUPPORTED
    assert ska(T=(1 << 30), B=0) == rd.ERR_UNSUPPORTED


def skadec(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, pos=FAKE, o=FAKE, N=2, H=3, dk=128, dv=128,
             window=256, scale=0.088, dtype=rd.BF16, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return rd.lib().sw_ska_decode_step(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["pos"], a["o"],
                                       a["N"], a["H"], a["dk"], a["dv"], a["window"], a["scale"],
                                       a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(kn=None), dict(vn=None), dict(kc=None), dict(vc=None), dict(o=None),
    dict(pos=None), dict(pos=FAKE + 2), dict(q=MISALIGNED), dict(kc=MISALIGNED), dict(ws=None),
    dict(ws_bytes=16), dict(N=-1), dict(H=-1), dict(window=0), dict(window=-5), dict(dk=7),
    dict(scale=0.0), dict(scale=float("nan")), dict(scale=float("inf")), dict(dtype=5),
    # launches of 2^32 work-items or more: N*H sequence-heads, or 256-slot
    # splits x heads, at 2^24
    dict(N=1 << 22, H=4), dict(N=1 << 13, H=16, window=1 << 19),
])
def test_swska_decode_rejects(kw):
    assert skadec(**kw) == rd.ERR_INVALID_ARG


def test_swska_decode_unsupported_and_empty():
    assert skadec(dk=128, dv=64) == rd.ERR_UNSUPPORTED
    assert skadec(dk=32, dv=32) == rd.ERR_UNSUPPORTED
    assert skadec(dtype=rd.F32) == rd.ERR_UNSUPPORTED
    assert skadec(N=0, q=None, ws=None) == rd.OK
    assert skadec(H=0, q=None, ws=None) == rd.OK


def test_swska_decode_workspace_query():
    # per (sequence, head) and 256-slot split: dv outputs + max + sum (+ 2 pad), fp32
    assert rd.sw_ska_decode_workspace_bytes(64, 16, 128, 128, 4096) == 64 * 16 * 16 * 132 * 4
    assert rd.sw_ska_decode_workspace_bytes(3, 5, 64, 64, 100) == 3 * 5 * 68 * 4
    assert rd.sw_ska_decode_workspace_bytes(3, 5, 64, 64, 257) == 3 * 5 * 2 * 68 * 4
    assert rd.sw_ska_decode_workspace_bytes(3, 5, 64, 32, 100) == 0      # unsupported
    assert rd.sw_ska_decode_workspace_bytes(3, 5, 64, 64, 0) == 0        # invalid window


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, tau=FAKE, S0=None, dO=FAKE, dST=None, dq=FAKE, dk_=FAKE,
             dv_=FAKE, dg=FAKE, dtau=FAKE, dS0=FAKE, B=1, H=2, T=40, dk=16, dv=32, dtype=rd.BF16,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return rd.lib().rodimus_scan_backward(a["q"], a["k"], a["v"], a["g"], a["tau"], a["S0"], a["dO"],
                                          a["dST"], a["dq"], a["dk_"], a["dv_"], a["dg"], a["dtau"],
                                          a["dS0"], a["B"], a["H"], a["T"], a["dk"], a["dv"],
                                          a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(g=None), dict(tau=None), dict(dO=None),
    dict(dq=None), dict(dk_=None), dict(dv_=None), dict(dg=None), dict(dtau=None),
    dict(q=MISALIGNED), dict(S0=MISALIGNED), dict(dST=MISALIGNED), dict(dS0=MISALIGNED),
    dict(ws=MISALIGNED), dict(ws=None), dict(ws_bytes=2 * 2 * 16 * 32 * 4 * 2 - 4),
    dict(B=-1), dict(H=-1), dict(T=-1), dict(dk=8), dict(dk=144), dict(dv=0), dict(dtype=2),
])
def test_scan_backward_rejects(kw):
    assert bwd(**kw) == rd.ERR_INVALID_ARG


def _mfma_bwd_workspace(B, H, T):
    """Workspace of the matrix-core backward (bf16, dk = dv = 128): bf16
    checkpoints of S and G every 32 tokens (32 KiB each), per-checkpoint decay
    factors, per-segment edges, the fallback list and 256 scratch pairs."""
    up = lambda x: (x + 255) // 256 * 256
    BH = B * H
    nck = -(-T // 32)
    nseg = max(1, min(nck, -(-256 // BH)))
    seg_ck = -(-nck // nseg)
    nseg = -(-nck // seg_ck)
    return (2 * up(BH * nck * 32768) + 2 * up(BH * nck * 512) + 2 * up(BH * nseg * 65536)
            + 2 * up(BH * nseg * 512) + 2 * up(BH * nseg * 32768) + up(4 * (1 + BH * nck))
            + 256 * 2 * 128 * 128 * 4)


def test_scan_backward_empty_and_workspace():
    assert bwd(B=0, q=None, ws=None) == rd.OK
    assert bwd(H=0, dq=None, ws=None) == rd.OK
    assert bwd(T=0, dS0=None, q=None, ws=None) == rd.OK     # nothing requested
    # generic path: two fp32 [dk,dv] states per (batch, head, 32-token chunk)
    assert rd.rodimus_scan_backward_workspace_bytes(1, 2, 40, 16, 32) == 2 * 2 * 2 * 16 * 32 * 4
    assert rd.rodimus_scan_backward_workspace_bytes(4, 16, 4096, 128, 128, rd.F32) == 2 * 64 * 128 * 128 * 128 * 4
    # matrix-core path (bf16, dk = dv = 128)
    for B, H, T in ((4, 16, 4096), (1, 16, 131072), (1, 1, 1), (3, 5, 100), (300, 1, 640)):
        assert rd.rodimus_scan_backward_workspace_bytes(B, H, T, 128, 128) == _mfma_bwd_workspace(B, H, T)
    assert rd.rodimus_scan_backward_workspace_bytes(1, 1, 0, 128, 128) == 0
    assert rd.rodimus_scan_backward_workspace_bytes(1, 1, 64, 8, 128) == 0   # invalid dk


def varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, tau=FAKE, S0=None, o=FAKE, S_T=None, cu=FAKE, N=3, H=2,
             total=100, maxlen=64, dk=128, dv=128, chunk=64, dtype=rd.BF16, ws=FAKE, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return rd.lib().rodimus_scan_prefill_varlen(a["q"], a["k"], a["v"], a["g"], a["tau"], a["S0"], a["o"],
                                                a["S_T"], a["cu"], a["N"], a["H"], a["total"], a["maxlen"],
                                                a["dk"], a["dv"], a["chunk"], a["dtype"], a["ws"],
                                                a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(o=None), dict(cu=None), dict(cu=FAKE + 2), dict(q=MISALIGNED), dict(S0=MISALIGNED),
    dict(N=-1), dict(H=-1), dict(total=-1), dict(maxlen=-1), dict(dk=8), dict(chunk=48), dict(dtype=3),
    dict(S0=FAKE, S_T=FAKE), dict(ws=MISALIGNED),
])
def test_scan_prefill_varlen_rejects(kw):
    assert varlen(**kw) == rd.ERR_INVALID_ARG


def test_scan_prefill_varlen_empty_and_workspace():
    assert varlen(N=0, q=None, cu=None) == rd.OK
    assert varlen(H=0, o=None, cu=None) == rd.OK
    assert varlen(maxlen=0, q=None, o=None) == rd.OK      # every sequence empty, nothing to copy
    assert varlen(total=0, q=None, o=None) == rd.OK
    # the segment plan of a packed batch is that of N sequences of the longest
    # length, plus the longest-first order of the sequences (int32, 256-byte
    # granules, for every N)
    for N, H, L, d, dt in ((3, 16, 4096, 128, rd.BF16), (64, 16, 448, 128, rd.BF16), (1, 1, 1, 128, rd.BF16),
                           (4096, 1, 8, 128, rd.BF16), (4097, 1, 8, 128, rd.BF16), (5, 3, 70, 32, rd.F32)):
        assert (rd.rodimus_scan_prefill_varlen_workspace_bytes(N, H, L, d, d, 64, dt)
                == rd.rodimus_scan_prefill_workspace_bytes(N, H, L, d, d, 64, dt) + _order_bytes(N))
    assert rd.rodimus_scan_prefill_varlen_workspace_bytes(3, 2, 64, 8, 128, 64, rd.BF16) == 0   # invalid dk
    # a workspace without room for the order is rejected
    need = rd.rodimus_scan_prefill_varlen_workspace_bytes(3, 2, 64, 128, 128, 64, rd.BF16)
    assert varlen(ws_bytes=need - 4) == rd.ERR_INVALID_ARG


def _order_bytes(N):
    return (4 * N + 255) // 256 * 256 if N > 0 else 0


def bwd_varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, tau=FAKE, S0=None, dO=FAKE, dST=None, dq=FAKE, dk_=FAKE,
             dv_=FAKE, dg=FAKE, dtau=FAKE, dS0=FAKE, cu=FAKE, N=3, H=2, total=100, maxlen=64, dk=128,
             dv=128, dtype=rd.BF16, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return rd.lib().rodimus_scan_backward_varlen(a["q"], a["k"], a["v"], a["g"], a["tau"], a["S0"], a["dO"],
                                                 a["dST"], a["dq"], a["dk_"], a["dv_"], a["dg"], a["dtau"],
                                                 a["dS0"], a["cu"], a["N"], a["H"], a["total"], a["maxlen"],
                                                 a["dk"], a["dv"], a["dtype"], a["ws"], a["ws_bytes"],
                                                 a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(dO=None), dict(dq=None), dict(dtau=None), dict(cu=None), dict(cu=FAKE + 2),
    dict(q=MISALIGNED), dict(S0=MISALIGNED), dict(dST=MISALIGNED), dict(dS0=MISALIGNED),
    dict(ws=MISALIGNED), dict(ws=None), dict(ws_bytes=1000),
    dict(N=-1), dict(H=-1), dict(total=-1), dict(maxlen=-1), dict(dk=8), dict(dv=144), dict(dtype=3),
])
def test_scan_backward_varlen_rejects(kw):
    assert bwd_varlen(**kw) == rd.ERR_INVALID_ARG


def test_scan_backward_varlen_empty_and_workspace():
    assert bwd_varlen(N=0, q=None, cu=None, ws=None) == rd.OK
    assert bwd_varlen(H=0, dq=None, cu=None, ws=None) == rd.OK
    assert bwd_varlen(maxlen=0, dS0=None, q=None, ws=None) == rd.OK   # every sequence empty, nothing requested
    assert bwd_varlen(total=0, dS0=None, q=None, ws=None) == rd.OK
    # the plan of a packed batch is that of N sequences of the longest length,
    # plus the longest-first order of the sequences
    for N, H, L, d, dt in ((3, 16, 4096, 128, rd.BF16), (64, 16, 1131, 128, rd.BF16), (1, 1, 1, 128, rd.BF16),
                           (5, 3, 70, 32, rd.F32), (4097, 1, 8, 128, rd.BF16)):
        assert (rd.rodimus_scan_backward_varlen_workspace_bytes(N, H, L, d, d, dt)
                == rd.rodimus_scan_backward_workspace_bytes(N, H, L, d, d, dt) + _order_bytes(N))
    need = rd.rodimus_scan_backward_varlen_workspace_bytes(3, 2, 64, 128, 128, rd.BF16)
    assert bwd_varlen(ws_bytes=need - 4) == rd.ERR_INVALID_ARG


# ---------------------------------------------------------------- launch sizes
# HIP refuses a launch of 2^32 work-items or more.  Each entry point computes
# its largest launch before doing anything and returns INVALID_ARG (instead of
# launching and reporting ERR_HIP).  A huge workspace is passed so that only the
# launch-size rule can reject these calls; no pointer is ever dereferenced.
HUGE_WS = 1 << 62


def test_prefill_rejects_a_grid_beyond_hip_limits():
    # matrix-core path: one 512-thread workgroup per (b,h) once B*H >= 256
    assert scan(B=1 << 13, H=1 << 10, T=64, dk=128, dv=128, ws=FAKE, ws_bytes=HUGE_WS) == rd.ERR_INVALID_ARG
    assert scan(B=1 << 12, H=1 << 11, T=64, dk=128, dv=128, chunk=32, ws=FAKE,
                ws_bytes=HUGE_WS) == rd.ERR_INVALID_ARG
    # vector path (fp32): one 64-thread wave per (b,h)
    assert scan(B=1 << 16, H=1 << 10, T=1, dk=16, dv=16, dtype=rd.F32, ws=FAKE,
                ws_bytes=HUGE_WS) == rd.ERR_INVALID_ARG
    # the packed form applies the same plan
    assert varlen(N=1 << 13, H=1 << 10, total=1 << 13, maxlen=64, ws=FAKE,
                  ws_bytes=HUGE_WS) == rd.ERR_INVALID_ARG


def test_backward_rejects_a_grid_beyond_hip_limits():
    # matrix-core gradient kernel: 8 work-items per token-head
    assert bwd(B=1, H=1 << 10, T=1 << 19, dk=128, dv=128, ws_bytes=HUGE_WS) == rd.ERR_INVALID_ARG
    # vector path: 256 threads per 32-token chunk of every (b,h)
    assert bwd(B=1, H=1 << 10, T=1 << 19, dk=16, dv=16, dtype=rd.F32, ws_bytes=HUGE_WS) == rd.ERR_INVALID_ARG
    assert bwd_varlen(N=1 << 10, H=1, total=1 << 19, maxlen=1 << 19, ws_bytes=HUGE_WS) == rd.ERR_INVALID_ARG


def test_decode_rejects_a_grid_beyond_hip_limits():
    # one workgroup of up to 256 threads per (sequence, head): N*H < 2^24
    assert decode(N=1 << 12, H=1 << 12) == rd.ERR_INVALID_ARG
    assert decode(N=1 << 24, H=1) == rd.ERR_INVALID_ARG
    assert decode(N=1 << 12, H=1 << 12, dk=128, dv=128) == rd.ERR_INVALID_ARG


def test_swska_rejects_a_grid_beyond_hip_limits():
    # one 512-thread workgroup per (b,h) and 256 query rows
    assert ska(B=1, H=1 << 10, T=1 << 21) == rd.ERR_INVALID_ARG
    # d = 64: 256 threads per 128 query rows
    assert ska(B=1, H=1 << 10, T=1 << 21, dk=64, dv=64) == rd.ERR_INVALID_ARG


# ------------------------------------------------- prefill without allocation
def scan_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, tau=FAKE, S0=None, o=FAKE, S_T=None, B=1, H=1, T=8,
             dk=16, dv=16, chunk=64, dtype=rd.BF16, stream=None)
    a.update(kw)
    return rd.lib().rodimus_scan_prefill_noalloc(a["q"], a["k"], a["v"], a["g"], a["tau"], a["S0"], a["o"],
                                                 a["S_T"], a["B"], a["H"], a["T"], a["dk"], a["dv"],
                                                 a["chunk"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(tau=None), dict(o=None), dict(q=MISALIGNED), dict(S0=MISALIGNED), dict(S_T=MISALIGNED),
    dict(B=-1), dict(T=-1), dict(dk=8), dict(dv=136), dict(chunk=8), dict(dtype=2), dict(S0=FAKE, S_T=FAKE),
    dict(B=1 << 13, H=1 << 10, T=64, dk=128, dv=128),      # grid beyond HIP's limit
])
def test_scan_noalloc_rejects_before_any_hip_call(kw):
    # the scratch array's address is looked up only after validation has passed
    assert scan_noalloc(**kw) == rd.ERR_INVALID_ARG


def test_scan_noalloc_empty_is_noop():
    assert scan_noalloc(B=0, q=None) == rd.OK
    assert scan_noalloc(T=0, q=None, o=None) == rd.OK


def test_scan_noalloc_scratch_covers_every_segment_plan():
    # the fixed array (34 MiB) holds the workspace of the largest segment plan
    # the prefill can make, so the no-allocation call never runs out of scratch
    worst = max(rd.rodimus_scan_prefill_workspace_bytes(1, bh, T, 128, 128, c, rd.BF16)
                for bh in (1, 2, 3, 5, 16, 17, 64, 100, 128, 255) for T in (4096, 32704, 131072, 8388607)
                for c in (32, 64))
    assert worst == 33684480 <= 34 << 20


# ------------------------------------------------- prefill with low-rank gates
def scan_lowrank(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, zg=FAKE, zt=FAKE, Ug=FAKE, bg=FAKE, Ut=FAKE, bt=FAKE, S0=None, o=FAKE,
             S_T=None, B=1, H=2, T=100, dk=128, dv=128, R=16, chunk=64, dtype=rd.BF16, ws=FAKE,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return rd.lib().rodimus_scan_prefill_lowrank(a["q"], a["k"], a["v"], a["zg"], a["zt"], a["Ug"], a["bg"],
                                                 a["Ut"], a["bt"], a["S0"], a["o"], a["S_T"], a["B"], a["H"],
                                                 a["T"], a["dk"], a["dv"], a["R"], a["chunk"], a["dtype"],
                                                 a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(v=None), dict(zg=None), dict(zt=None), dict(Ug=None), dict(bg=None), dict(Ut=None),
    dict(bt=None), dict(o=None), dict(zg=MISALIGNED), dict(bt=MISALIGNED), dict(S0=MISALIGNED),
    dict(S0=FAKE, S_T=FAKE), dict(B=-1), dict(T=-1), dict(R=0), dict(R=-16), dict(chunk=48), dict(dtype=5),
    dict(ws=None), dict(ws_bytes=1000),
    dict(B=1 << 13, H=1 << 10, T=64, ws_bytes=1 << 62),         # grid beyond HIP's limit
])
def test_scan_lowrank_rejects(kw):
    assert scan_lowrank(**kw) == rd.ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(dtype=rd.F32), dict(dk=64), dict(dv=64), dict(R=8), dict(R=32), dict(chunk=16),
    dict(T=1 << 23),
])
def test_scan_lowrank_unsupported(kw):
    assert scan_lowrank(**kw) == rd.ERR_UNSUPPORTED


def test_scan_lowrank_empty_is_noop():
    assert scan_lowrank(B=0, q=None) == rd.OK
    assert scan_lowrank(T=0, q=None, zg=None, o=None) == rd.OK
