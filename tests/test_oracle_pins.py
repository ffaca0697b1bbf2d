"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than itself: a brute-force
quadratic form, a reduction to a textbook routine, a closed form, a special gate
setting whose result is known, or a library routine (torch CPU SDPA).  Chosen so
that a dropped term, a wrong sign, a wrong index or a transposed operand in the
oracle fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.chunk_model import chunked_scan, gates_power_form, segment_scan

RNG = np.random.default_rng(1234)


def rand_inputs(B, H, T, dk, dv, gate_mu=0.0, gate_sigma=1.0, rng=RNG):
    q = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, H, T, dv))
    g = gate_mu + gate_sigma * rng.standard_normal((B, H, T, dk))
    th = gate_mu + gate_sigma * rng.standard_normal((B, H, T, dk))
    return q, k, v, g, th


def relerr(x, r):
    return np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300)


# ------------------------------------------------------------------ gate map

def test_gates_match_power_form():
    """log-space softplus form == sigmoid(g)**sigmoid(theta) and (1-sigmoid(g))**sigmoid(theta)."""
    g = np.linspace(-30, 30, 241)
    th = np.linspace(-20, 20, 241)[::-1]
    la, lb = oracle.gates(g, th)
    a, b = gates_power_form(g, th)
    np.testing.assert_allclose(np.exp(la), a, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(np.exp(lb), b, rtol=1e-13, atol=1e-300)


def test_gates_special_values():
    # tau = sigmoid(+inf) = 1: an exponential moving average, a + beta = 1; g = 0 -> 1/2 each.
    g = np.array([0.0, 2.0, -3.0, 7.5])
    la, lb = oracle.gates(g, np.full(4, np.inf))
    np.testing.assert_allclose(np.exp(la) + np.exp(lb), 1.0, rtol=1e-15)
    assert np.exp(la[0]) == pytest.approx(0.5, rel=1e-15)
    # tau = sigmoid(-inf) = 0: no decay, no input gating (plain linear attention).
    la, lb = oracle.gates(g, np.full(4, -np.inf))
    assert np.all(la == 0.0) and np.all(lb == 0.0)
    # tempered_gate_init 0.5 (theta = 0): a = sqrt(sigmoid(g)).
    la, lb = oracle.gates(g, np.zeros(4))
    np.testing.assert_allclose(np.exp(la), np.sqrt(1 / (1 + np.exp(-g))), rtol=1e-14)
    # selection: large g keeps the past (a -> 1, beta -> 0); small g resets (a -> 0, beta -> 1).
    la, lb = oracle.gates(np.array([40.0, -40.0]), np.array([40.0, 40.0]))
    assert np.exp(la[0]) > 1 - 1e-15 and np.exp(lb[0]) < 1e-17
    assert np.exp(la[1]) < 1e-17 and np.exp(lb[1]) > 1 - 1e-15
    # monotone: a increases with g, beta decreases with g.
    g = np.linspace(-5, 5, 101)
    la, lb = oracle.gates(g, np.full_like(g, 0.3))
    assert np.all(np.diff(la) > 0) and np.all(np.diff(lb) < 0)


# ------------------------------------------------------------------ the scan

def brute_force(q, k, v, g, th, S0=None):
    """o_t = sum_{s<=t} (q_t * prod_{r=s+1..t} a_r * beta_s * k_s) . v_s
             + (q_t * prod_{r<=t} a_r) . S0     (per (b,h), O(T^2) explicit products)."""
    a, beta = gates_power_form(g, th)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = np.zeros(dv)
                for s in range(t + 1):
                    decay = np.prod(a[b, h, s + 1:t + 1], axis=0)
                    w = q[b, h, t] * decay * beta[b, h, s] * k[b, h, s]
                    acc += w.sum() * v[b, h, s]
                if S0 is not None:
                    decay = np.prod(a[b, h, :t + 1], axis=0)
                    acc += (q[b, h, t] * decay) @ S0[b, h]
                o[b, h, t] = acc
    return o


@pytest.mark.parametrize("with_s0", [False, True])
def test_scan_vs_brute_force(with_s0):
    B, H, T, dk, dv = 2, 2, 24, 5, 3
    q, k, v, g, th = rand_inputs(B, H, T, dk, dv)
    S0 = RNG.standard_normal((B, H, dk, dv)) if with_s0 else None
    o, ST = oracle.scan(q, k, v, g, th, S0)
    ob = brute_force(q, k, v, g, th, S0)
    assert relerr(o, ob) < 1e-12


def test_scan_final_state_brute_force():
    """S_T = sum_s diag(prod_{r>s} a_r) (beta_s k_s)^T v_s + diag(prod a) S0."""
    B, H, T, dk, dv = 1, 1, 17, 4, 6
    q, k, v, g, th = rand_inputs(B, H, T, dk, dv)
    S0 = RNG.standard_normal((B, H, dk, dv))
    _, ST = oracle.scan(q, k, v, g, th, S0)
    a, beta = gates_power_form(g, th)
    S = np.prod(a[0, 0], axis=0)[:, None] * S0[0, 0]
    for s in range(T):
        S = S + (np.prod(a[0, 0, s + 1:], axis=0) * beta[0, 0, s] * k[0, 0, s])[:, None] * v[0, 0, s][None, :]
    assert relerr(ST[0, 0], S) < 1e-13


def test_reduction_to_causal_linear_attention():
    """theta = -inf gives a = beta = 1: o_t = q_t . sum_{s<=t} k_s^T v_s (linear attention
    with identity feature map, MiniCPM-SALA blog section 2.2)."""
    B, H, T, dk, dv = 2, 3, 40, 8, 7
    q, k, v, g, _ = rand_inputs(B, H, T, dk, dv)
    th = np.full_like(g, -np.inf)
    o, ST = oracle.scan(q, k, v, g, th)
    KV = np.cumsum(k[..., :, None] * v[..., None, :], axis=2)  # [B,H,T,dk,dv]
    ref = np.einsum("bhti,bhtij->bhtj", q, KV)
    assert relerr(o, ref) < 1e-13
    assert relerr(ST, KV[:, :, -1]) < 1e-13


def test_reset_gates():
    """g = -40, theta = +40: a ~ 4e-18, beta ~ 1 -> o_t = (q_t . k_t) v_t, S_T = k_T^T v_T."""
    B, H, T, dk, dv = 1, 2, 12, 6, 5
    q, k, v, _, _ = rand_inputs(B, H, T, dk, dv)
    g = np.full_like(q, -40.0)
    th = np.full_like(q, 40.0)
    S0 = RNG.standard_normal((B, H, dk, dv))
    o, ST = oracle.scan(q, k, v, g, th, S0)
    ref = (q * k).sum(-1)[..., None] * v
    assert relerr(o, ref) < 1e-14
    assert relerr(ST, k[:, :, -1, :, None] * v[:, :, -1, None, :]) < 1e-14


def test_skip_gates():
    """g = +40, theta = +40: a ~ 1, beta ~ 4e-18 -> the state is frozen at S0."""
    B, H, T, dk, dv = 1, 2, 12, 6, 5
    q, k, v, _, _ = rand_inputs(B, H, T, dk, dv)
    g = np.full_like(q, 40.0)
    th = np.full_like(q, 40.0)
    S0 = RNG.standard_normal((B, H, dk, dv))
    o, ST = oracle.scan(q, k, v, g, th, S0)
    assert relerr(o, np.einsum("bhti,bhij->bhtj", q, S0)) < 1e-14
    assert relerr(ST, S0) < 1e-14


@pytest.mark.parametrize("gval,thval", [(0.7, 0.0), (-1.3, 2.0), (2.5, -1.0)])
def test_geometric_closed_form(gval, thval):
    """Constant gates, k_t = q_t = e_i, v_t = 1: o_t = beta (1 - a^{t+1}) / (1 - a)."""
    T, dk, dv, i = 50, 4, 3, 2
    q = np.zeros((1, 1, T, dk))
    q[..., i] = 1.0
    k = q.copy()
    v = np.ones((1, 1, T, dv))
    g = np.full((1, 1, T, dk), gval)
    th = np.full((1, 1, T, dk), thval)
    o, ST = oracle.scan(q, k, v, g, th)
    s = 1 / (1 + np.exp(-gval))
    tau = 1 / (1 + np.exp(-thval))
    a, beta = s ** tau, (1 - s) ** tau
    t = np.arange(T)
    ref = beta * (1 - a ** (t + 1)) / (1 - a)
    np.testing.assert_allclose(o[0, 0, :, 0], ref, rtol=1e-13)
    np.testing.assert_allclose(o[0, 0], np.repeat(ref[:, None], dv, 1), rtol=1e-13)
    assert np.all(np.delete(ST[0, 0], i, axis=0) == 0.0)


def test_linearity():
    B, H, T, dk, dv = 1, 2, 30, 6, 4
    q, k, v, g, th = rand_inputs(B, H, T, dk, dv)
    v2 = RNG.standard_normal(v.shape)
    S0 = RNG.standard_normal((B, H, dk, dv))
    S1 = RNG.standard_normal((B, H, dk, dv))
    o1, s1 = oracle.scan(q, k, v, g, th, S0)
    o2, s2 = oracle.scan(q, k, v2, g, th, S1)
    o3, s3 = oracle.scan(q, k, 2 * v - 3 * v2, g, th, 2 * S0 - 3 * S1)
    assert relerr(o3, 2 * o1 - 3 * o2) < 1e-12
    assert relerr(s3, 2 * s1 - 3 * s2) < 1e-12
    o4, _ = oracle.scan(-2.5 * q, k, v, g, th, S0)
    assert relerr(o4, -2.5 * o1) < 1e-14


def test_split_resume():
    B, H, T, dk, dv = 2, 2, 37, 5, 6
    q, k, v, g, th = rand_inputs(B, H, T, dk, dv)
    o, ST = oracle.scan(q, k, v, g, th)
    T1 = 15
    oa, Sa = oracle.scan(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], g[:, :, :T1], th[:, :, :T1])
    ob, Sb = oracle.scan(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], g[:, :, T1:], th[:, :, T1:], Sa)
    assert relerr(np.concatenate([oa, ob], axis=2), o) < 1e-14
    assert relerr(Sb, ST) < 1e-14


def test_threads_identical():
    q, k, v, g, th = rand_inputs(3, 5, 33, 8, 8)
    o1, s1 = oracle.scan(q, k, v, g, th, nthreads=1)
    o4, s4 = oracle.scan(q, k, v, g, th, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)


def test_decode_steps_equal_scan():
    N, H, T, dk, dv = 3, 2, 20, 6, 5
    q, k, v, g, th = rand_inputs(N, H, T, dk, dv)
    S0 = RNG.standard_normal((N, H, dk, dv))
    o, ST = oracle.scan(q, k, v, g, th, S0)
    S = S0.copy()
    for t in range(T):
        ot, S = oracle.decode(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], th[:, :, t], S)
        assert relerr(ot, o[:, :, t]) < 1e-14
    assert relerr(S, ST) < 1e-14


def test_decode_geometric():
    """Identical inputs n times from S = 0: S_n = diag(beta (1-a^n)/(1-a)) k v^T."""
    N, H, dk, dv, n = 1, 1, 5, 4, 9
    q = RNG.standard_normal((N, H, dk))
    k = RNG.standard_normal((N, H, dk))
    v = RNG.standard_normal((N, H, dv))
    g = RNG.standard_normal((N, H, dk))
    th = RNG.standard_normal((N, H, dk))
    S = np.zeros((N, H, dk, dv))
    for _ in range(n):
        _, S = oracle.decode(q, k, v, g, th, S)
    a, beta = gates_power_form(g, th)
    ref = (beta * (1 - a ** n) / (1 - a) * k)[..., None] * v[..., None, :]
    assert relerr(S, ref) < 1e-13


# ------------------------------------------------------ chunked-form pins

@pytest.mark.parametrize("C", [1, 2, 3, 7, 16, 32, 64, 100])
def test_chunked_form_matches_sequential(C):
    B, H, T, dk, dv = 1, 2, 100, 8, 6
    q, k, v, g, th = rand_inputs(B, H, T, dk, dv)
    S0 = RNG.standard_normal((B, H, dk, dv))
    o, ST = oracle.scan(q, k, v, g, th, S0)
    oc, STc, _ = chunked_scan(q, k, v, g, th, C, S0)
    assert relerr(oc, o) < 1e-11
    assert relerr(STc, ST) < 1e-11


def test_chunked_form_extreme_gates_take_fallback():
    """Mixed-sign extreme logits drive the chunk decay span past the factorised
    form's range; the fallback keeps the chunked form equal to the definition."""
    B, H, T, dk, dv = 1, 1, 128, 8, 4
    q, k, v, _, _ = rand_inputs(B, H, T, dk, dv)
    g = RNG.choice([-8.0, 8.0], size=q.shape)
    th = RNG.choice([-2.0, 4.0], size=q.shape)
    o, ST = oracle.scan(q, k, v, g, th)
    oc, STc, nfb = chunked_scan(q, k, v, g, th, 64)
    assert nfb > 0
    assert relerr(oc, o) < 1e-11 and relerr(STc, ST) < 1e-11


@pytest.mark.parametrize("G", [1, 2, 3, 5])
def test_segment_form_matches_sequential(G):
    B, H, T, dk, dv = 1, 2, 150, 6, 5
    q, k, v, g, th = rand_inputs(B, H, T, dk, dv, gate_mu=2.0)
    S0 = RNG.standard_normal((B, H, dk, dv))
    o, ST = oracle.scan(q, k, v, g, th, S0)
    os_, STs = segment_scan(q, k, v, g, th, 16, G, S0)
    assert relerr(os_, o) < 1e-11 and relerr(STs, ST) < 1e-11


# ------------------------------------------------------------------ SW-SKA

def sdpa_ref(q, k_shared, v, window):
    """torch CPU scaled_dot_product_attention with K replicated over heads and a
    band mask (s in [t-w+1, t])."""
    B, H, T, dk = q.shape
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k_shared)[:, None].expand(B, H, T, dk).contiguous()
    vt = torch.from_numpy(v)
    t = torch.arange(T)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - window)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask).numpy()


@pytest.mark.parametrize("window", [1, 2, 5, 16, 33, 64, 1000])
def test_swska_vs_sdpa(window):
    B, H, T, dk, dv = 2, 3, 64, 16, 8
    q = RNG.standard_normal((B, H, T, dk))
    k = RNG.standard_normal((B, T, dk))
    v = RNG.standard_normal((B, H, T, dv))
    o = oracle.swska(q, k, v, window)
    assert relerr(o, sdpa_ref(q, k, v, window)) < 1e-12


def test_swska_full_window_is_causal_sdpa():
    B, H, T, dk, dv = 1, 4, 50, 8, 8
    q = RNG.standard_normal((B, H, T, dk))
    k = RNG.standard_normal((B, T, dk))
    v = RNG.standard_normal((B, H, T, dv))
    o = oracle.swska(q, k, v, T + 10)
    kt = torch.from_numpy(k)[:, None].expand(B, H, T, dk).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, torch.from_numpy(v), is_causal=True).numpy()
    assert relerr(o, ref) < 1e-12


def test_swska_window_one_is_identity():
    q = RNG.standard_normal((1, 2, 20, 8))
    k = RNG.standard_normal((1, 20, 8))
    v = RNG.standard_normal((1, 2, 20, 4))
    assert np.array_equal(oracle.swska(q, k, v, 1), v)


def test_swska_constant_key_is_window_mean():
    B, H, T, dk, dv, w = 1, 2, 30, 4, 3, 7
    q = RNG.standard_normal((B, H, T, dk))
    k = np.tile(RNG.standard_normal((1, 1, dk)), (B, T, 1))
    v = RNG.standard_normal((B, H, T, dv))
    o = oracle.swska(q, k, v, w)
    ref = np.stack([v[:, :, max(0, t - w + 1):t + 1].mean(axis=2) for t in range(T)], axis=2)
    assert relerr(o, ref) < 1e-14


def test_swska_shared_key_per_head_values():
    """Heads see the same keys (same weights for equal q) but their own values."""
    B, H, T, dk, dv, w = 1, 3, 25, 6, 5, 9
    q1 = RNG.standard_normal((B, 1, T, dk))
    q = np.repeat(q1, H, axis=1)
    k = RNG.standard_normal((B, T, dk))
    v = RNG.standard_normal((B, H, T, dv))
    o = oracle.swska(q, k, v, w)
    o_single = oracle.swska(q1, k, v[:, :1].copy(), w)
    assert relerr(o[:, :1], o_single) < 1e-15
    assert not np.allclose(o[:, 0], o[:, 1])


def test_swska_row_subset():
    B, H, T, dk, dv, w = 1, 2, 40, 8, 4, 10
    q = RNG.standard_normal((B, H, T, dk))
    k = RNG.standard_normal((B, T, dk))
    v = RNG.standard_normal((B, H, T, dv))
    full = oracle.swska(q, k, v, w, nthreads=3)
    rows = np.array([0, 5, 39, 40, 79])
    part = oracle.swska(q, k, v, w, rows=rows)
    flat_f = full.reshape(-1, dv)
    flat_p = part.reshape(-1, dv)
    assert np.array_equal(flat_p[rows], flat_f[rows])
    assert np.isnan(flat_p[1]).all()


# ------------------------------------------------------------------ golden

def test_golden_fixture_reproduced():
    """Regression lock: tests/golden/oracle_tiny.json (written by
    tests/golden/make_golden.py from the oracle) is reproduced exactly."""
    import json
    import os
    rec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")))
    a = {k: np.array(rec[k]) for k in ("q", "k", "v", "g", "theta", "S0", "o", "S_T")}
    o, ST = oracle.scan(a["q"], a["k"], a["v"], a["g"], a["theta"], a["S0"])
    np.testing.assert_allclose(o, a["o"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(ST, a["S_T"], rtol=1e-14, atol=1e-15)
    la, lb = oracle.gates(a["g"], a["theta"])
    np.testing.assert_allclose(la, rec["log_a"], rtol=1e-14)
    np.testing.assert_allclose(lb, rec["log_beta"], rtol=1e-14)
    os_ = oracle.swska(np.array(rec["swska_q"]), np.array(rec["swska_k"]), np.array(rec["swska_v"]),
                       rec["swska_window"])
    np.testing.assert_allclose(os_, rec["swska_o"], rtol=1e-14, atol=1e-15)
