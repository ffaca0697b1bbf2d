"""fp64 CPU oracle for the Rodimus* token mixer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The product path (the HIP library and its binding) never
does, and shares no code with it.

The arithmetic lives in ``rodimus_oracle.c`` (plain sequential fp64 loops); this
module compiles it with gcc and wraps it with numpy arrays.  What each function
computes, and the passages it follows, are stated in the C file's header:

* :func:`gates`  -- the DDTS gate map (our reading; the pages do not print it),
* :func:`scan`   -- the recurrence S_t = diag(a_t) S_{t-1} + (beta_t*k_t)^T v_t,
  o_t = q_t S_t, token by token,
* :func:`decode` -- one step of the same recurrence on a persistent state,
* :func:`swska`  -- sliding-window attention with one key matrix shared by all
  heads, dense softmax per query row,
* :func:`lowrank_gate_logits` / :func:`scan_lowrank` -- gate logits from
  rank-R factor rows shared by the heads (our reading of the gates' learnable
  weights), and the recurrence on them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rodimus_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp,
                               _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_gates.argtypes = [dp, dp, ctypes.c_size_t, dp, dp]
        lib.oracle_gates.restype = None
        lib.oracle_scan.argtypes = [ctypes.c_int] * 5 + [dp] * 6 + [dp, dp, ctypes.c_int]
        lib.oracle_scan.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [ctypes.c_int] * 4 + [dp] * 6 + [dp, dp]
        lib.oracle_scan_backward.argtypes = [ctypes.c_int] * 5 + [dp] * 14 + [ctypes.c_int]
        lib.oracle_scan_backward.restype = ctypes.c_int
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_swska.argtypes = ([ctypes.c_int] * 6 + [ctypes.c_double] + [dp] * 4 +
                                     [ctypes.POINTER(ctypes.c_longlong), ctypes.c_longlong,
                                      ctypes.c_int])
        lib.oracle_swska.restype = ctypes.c_int
        lib.oracle_lowrank_gate_logits.argtypes = [ctypes.c_int] * 5 + [dp] * 8
        lib.oracle_lowrank_gate_logits.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def gates(g, theta):
    """Return (log a, log beta), elementwise, fp64."""
    g = _f64(g)
    theta = _f64(theta)
    assert g.shape == theta.shape
    la = np.empty_like(g)
    lb = np.empty_like(g)
    _load().oracle_gates(_ptr(g), _ptr(theta), g.size, _ptr(la), _ptr(lb))
    return la, lb


def scan(q, k, v, g, theta, S0=None, nthreads: int = 1):
    """Sequential recurrence.  q,k,g,theta: [B,H,T,dk]; v: [B,H,T,dv];
    S0: [B,H,dk,dv] or None.  Returns (o [B,H,T,dv], S_T [B,H,dk,dv]) in fp64."""
    q, k, v, g, theta = (_f64(x) for x in (q, k, v, g, theta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    for x in (k, g, theta):
        assert x.shape == q.shape
    assert v.shape == (B, H, T, dv)
    if S0 is not None:
        S0 = _f64(S0)
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, H, T, dv))
    ST = np.empty((B, H, dk, dv))
    rc = _load().oracle_scan(B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(theta),
                             _ptr(S0), _ptr(o), _ptr(ST), int(nthreads))
    assert rc == 0
    return o, ST


def lowrank_gate_logits(zg, zt, Ug, bg, Ut, bt, H=None):
    """Gate logits from rank-R factor rows shared by the heads (our reading of
    the gates' learnable weights; see the C file):  g = silu(zg) Ug^T + bg,
    theta = zt Ut^T + bt per head.  zg, zt: [B,T,R]; Ug, Ut: [H,dk,R];
    bg, bt: [H,dk].  Returns (g, theta) [B,H,T,dk] in fp64."""
    zg, zt, Ug, bg, Ut, bt = (_f64(x) for x in (zg, zt, Ug, bg, Ut, bt))
    B, T, R = zg.shape
    H, dk, R2 = Ug.shape
    assert R2 == R and zt.shape == zg.shape and Ut.shape == Ug.shape
    assert bg.shape == (H, dk) and bt.shape == (H, dk)
    g = np.empty((B, H, T, dk))
    th = np.empty((B, H, T, dk))
    rc = _load().oracle_lowrank_gate_logits(B, H, T, dk, R, _ptr(zg), _ptr(zt), _ptr(Ug), _ptr(bg), _ptr(Ut),
                                            _ptr(bt), _ptr(g), _ptr(th))
    assert rc == 0
    return g, th


def scan_lowrank(q, k, v, zg, zt, Ug, bg, Ut, bt, S0=None, nthreads: int = 1):
    """The recurrence with gate logits from rank-R factors: lowrank_gate_logits
    followed by scan.  Returns (o, S_T) in fp64."""
    g, th = lowrank_gate_logits(zg, zt, Ug, bg, Ut, bt)
    return scan(q, k, v, g, th, S0=S0, nthreads=nthreads)


def scan_backward(q, k, v, g, theta, dO, S0=None, dST=None, nthreads: int = 1):
    """Gradients of sum(dO * o) + sum(dST * S_T) of the sequential recurrence
    with respect to q, k, v, g, theta and S0.  Returns a dict of fp64 arrays
    dq, dk, dv, dg, dtheta (shaped like the inputs) and dS0 [B,H,dk,dv]."""
    q, k, v, g, theta, dO = (_f64(x) for x in (q, k, v, g, theta, dO))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    for x in (k, g, theta):
        assert x.shape == q.shape
    assert v.shape == (B, H, T, dv) and dO.shape == (B, H, T, dv)
    if S0 is not None:
        S0 = _f64(S0)
        assert S0.shape == (B, H, dk, dv)
    if dST is not None:
        dST = _f64(dST)
        assert dST.shape == (B, H, dk, dv)
    out = dict(dq=np.empty_like(q), dk=np.empty_like(k), dv=np.empty_like(v), dg=np.empty_like(g),
               dtheta=np.empty_like(theta), dS0=np.empty((B, H, dk, dv)))
    rc = _load().oracle_scan_backward(B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                      _ptr(theta), _ptr(S0), _ptr(dO), _ptr(dST), _ptr(out["dq"]),
                                      _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                                      _ptr(out["dtheta"]), _ptr(out["dS0"]), int(nthreads))
    assert rc == 0
    return out


def decode(q, k, v, g, theta, S):
    """One recurrent step.  q,k,g,theta: [N,H,dk]; v: [N,H,dv]; S: [N,H,dk,dv].
    Returns (o [N,H,dv], S' [N,H,dk,dv]); the input S is not modified."""
    q, k, v, g, theta, S = (_f64(x) for x in (q, k, v, g, theta, S))
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert S.shape == (N, H, dk, dv)
    o = np.empty((N, H, dv))
    S_out = np.empty_like(S)
    rc = _load().oracle_decode(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(theta),
                               _ptr(S), _ptr(o), _ptr(S_out))
    assert rc == 0
    return o, S_out


def swska(q, k_shared, v, window: int, scale=None, rows=None, nthreads: int = 1):
    """Sliding-window shared-key attention.  q: [B,H,T,dk]; k_shared: [B,T,dk];
    v: [B,H,T,dv].  ``rows``: optional flat indices (b*H+h)*T+t of the query rows
    to compute; the others are returned as NaN.  Returns o [B,H,T,dv] fp64."""
    q, k_shared, v = (_f64(x) for x in (q, k_shared, v))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k_shared.shape == (B, T, dk) and v.shape == (B, H, T, dv)
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    o = np.full((B, H, T, dv), np.nan)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rp = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong))
        nr = rows.size
    else:
        rp, nr = None, 0
    rc = _load().oracle_swska(B, H, T, dk, dv, int(window), float(scale), _ptr(q), _ptr(k_shared),
                              _ptr(v), _ptr(o), rp, nr, int(nthreads))
    assert rc == 0
    return o
