"""fp64 numpy model of the chunked and segment-parallel forms of the scan.

This is a test pin, not part of either implementation: it writes out, in
plain numpy, the chunkwise algebra that the HIP kernels use, so that the test
suite can check on the CPU that the algebra reproduces the sequential
definition for every chunk size C (the chunkwise-parallel form is the same
model as the recurrence: Rodimus block paragraph of "ICLR 2025 | Rodimus*: ..."
(CodeFuse), which trains with a chunkwise-parallel, sub-quadratic algorithm and
infers with the recurrent form).

Per chunk of L <= C tokens entering with state S, with Lam[t] the inclusive
cumulative sum of log a inside the chunk:
    Qt = q * exp(Lam)               Kh = k * exp(log beta - Lam)
    Kb = k * exp(log beta + Lam[L-1] - Lam)
    O  = Qt S + tril(Qt Kh^T) V
    S' = diag(exp(Lam[L-1])) S + Kb^T V
The factorised form needs exp(-Lam) to stay finite; when the chunk's decay span
max_i(-Lam[L-1, i]) exceeds ``span_limit`` the chunk is processed token by token
instead (same result, no overflow).
"""
import numpy as np
from scipy.special import expit as sigmoid  # library logistic function, accurate for both signs


def gates_power_form(g, theta):
    """a = s^tau, beta = (1-s)^tau with s = sigmoid(g), tau = sigmoid(theta)."""
    g = np.asarray(g, dtype=np.float64)
    s = sigmoid(g)
    one_minus_s = sigmoid(-g)  # 1 - s without cancellation
    tau = sigmoid(np.asarray(theta, dtype=np.float64))
    return s ** tau, one_minus_s ** tau


def _log_gates(g, theta):
    # log a = tau * log(s), log beta = tau * log(1 - s), with log s = -logaddexp(0, -g)
    tau = sigmoid(theta)
    la = -tau * np.logaddexp(0.0, -g)
    lb = -tau * np.logaddexp(0.0, g)
    return la, lb


def chunk_step(q, k, v, la, lb, S, span_limit=80.0):
    """One chunk for one (b,h): q,k,la,lb [L,dk], v [L,dv], S [dk,dv]."""
    Lam = np.cumsum(la, axis=0)
    span = -Lam[-1]
    if span.max() <= span_limit:
        Qt = q * np.exp(Lam)
        Kh = k * np.exp(lb - Lam)
        Kb = k * np.exp(lb + Lam[-1] - Lam)
        A = np.tril(Qt @ Kh.T)
        O = Qt @ S + A @ v
        S = np.exp(Lam[-1])[:, None] * S + Kb.T @ v
        return O, S, True
    O = np.empty((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        S = np.exp(la[t])[:, None] * S + (np.exp(lb[t]) * k[t])[:, None] * v[t][None, :]
        O[t] = q[t] @ S
    return O, S, False


def chunked_scan(q, k, v, g, theta, C, S0=None, span_limit=80.0):
    """Chunked form over [B,H,T,*] inputs; returns (o, S_T, n_fallback_chunks)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    la, lb = _log_gates(np.asarray(g, np.float64), np.asarray(theta, np.float64))
    o = np.zeros((B, H, T, dv))
    ST = np.zeros((B, H, dk, dv))
    nfb = 0
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for c0 in range(0, T, C):
                c1 = min(T, c0 + C)
                O, S, ok = chunk_step(q[b, h, c0:c1], k[b, h, c0:c1], v[b, h, c0:c1],
                                      la[b, h, c0:c1], lb[b, h, c0:c1], S, span_limit)
                o[b, h, c0:c1] = O
                nfb += (not ok)
            ST[b, h] = S
    return o, ST, nfb


def segment_scan(q, k, v, g, theta, C, G, S0=None):
    """Segment-parallel form: split T into G segments; phase 1 computes each
    segment's local end state (from zero) and total log decay; phase 2 combines
    them left to right into each segment's incoming state; phase 3 reruns each
    segment from its incoming state.  Returns (o, S_T)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    la, lb = _log_gates(np.asarray(g, np.float64), np.asarray(theta, np.float64))
    bounds = np.linspace(0, T, G + 1).astype(int)
    o = np.zeros((B, H, T, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            Sloc, Atot = [], []
            for j in range(G):
                s0, s1 = bounds[j], bounds[j + 1]
                S = np.zeros((dk, dv))
                for c0 in range(s0, s1, C):
                    c1 = min(s1, c0 + C)
                    _, S, _ = chunk_step(q[b, h, c0:c1], k[b, h, c0:c1], v[b, h, c0:c1],
                                         la[b, h, c0:c1], lb[b, h, c0:c1], S)
                Sloc.append(S)
                Atot.append(la[b, h, s0:s1].sum(axis=0))
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for j in range(G):
                s0, s1 = bounds[j], bounds[j + 1]
                Sj = S
                for c0 in range(s0, s1, C):
                    c1 = min(s1, c0 + C)
                    O, Sj, _ = chunk_step(q[b, h, c0:c1], k[b, h, c0:c1], v[b, h, c0:c1],
                                          la[b, h, c0:c1], lb[b, h, c0:c1], Sj)
                    o[b, h, c0:c1] = O
                S = np.exp(Atot[j])[:, None] * S + Sloc[j]
            ST[b, h] = S
    return o, ST
