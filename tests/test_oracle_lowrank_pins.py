"""Pins of the oracle's low-rank gate logits (CPU only).

oracle.lowrank_gate_logits computes, per head h and key channel c, from
rank-R factor rows shared by the heads (our reading of the gates' learnable
weights; the CodeFuse article's Rodimus block paragraph and section 3 of the
Rodimus* deployment blog, which names SiLU as the selection gate's activation):

    g[b,h,t,c]     = sum_r silu(z_g[b,t,r]) U_g[h,c,r]   + b_g[h,c]
    theta[b,h,t,c] = sum_r      z_tau[b,t,r] U_tau[h,c,r] + b_tau[h,c]

The pins below tie it to things other than its own C loops: library routines
(scipy's logistic function and numpy's tensor contraction), the identity
silu(x) = x (1 + tanh(x/2)) / 2, exact special cases, the symmetries of the
definition, and -- through the scan -- the geometric closed form of constant
gates."""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle


def _factors(seed, B=2, H=3, T=7, dk=5, R=4, bias=True):
    rng = np.random.default_rng(seed)
    zg = rng.standard_normal((B, T, R)) * 1.5
    zt = rng.standard_normal((B, T, R))
    Ug = rng.standard_normal((H, dk, R)) / np.sqrt(R)
    Ut = rng.standard_normal((H, dk, R)) / np.sqrt(R)
    bg = rng.standard_normal((H, dk)) * 0.5 if bias else np.zeros((H, dk))
    bt = rng.standard_normal((H, dk)) * 0.5 if bias else np.zeros((H, dk))
    return zg, zt, Ug, bg, Ut, bt


@pytest.mark.parametrize("seed,shape", [(1, (2, 3, 7, 5, 4)), (2, (1, 1, 1, 1, 1)), (3, (3, 2, 9, 16, 16))])
def test_lowrank_logits_match_numpy_contraction(seed, shape):
    B, H, T, dk, R = shape
    zg, zt, Ug, bg, Ut, bt = _factors(seed, B, H, T, dk, R)
    g, th = oracle.lowrank_gate_logits(zg, zt, Ug, bg, Ut, bt)
    act = zg * expit(zg)
    g_ref = np.einsum("btr,hcr->bhtc", act, Ug) + bg[None, :, None, :]
    th_ref = np.einsum("btr,hcr->bhtc", zt, Ut) + bt[None, :, None, :]
    assert np.allclose(g, g_ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(th, th_ref, rtol=1e-13, atol=1e-13)


def test_lowrank_silu_values_from_the_tanh_identity():
    # rank 1, U_g = 1, no bias: g is silu(z) itself
    xs = np.array([0.0, 1.0, -1.0, 2.0, -3.0, 0.5, -0.25, 10.0, -12.0, 40.0, -40.0])
    zg = xs.reshape(1, -1, 1)
    zt = np.zeros_like(zg)
    g, th = oracle.lowrank_gate_logits(zg, zt, np.ones((1, 1, 1)), np.zeros((1, 1)), np.ones((1, 1, 1)),
                                       np.zeros((1, 1)))
    ref = np.array([x * (1.0 + math.tanh(x / 2.0)) / 2.0 for x in xs])
    # (1 + tanh(x/2)) cancels to 0 in fp64 for very negative x: absolute tolerance there
    assert np.allclose(g[0, 0, :, 0], ref, rtol=1e-14, atol=1e-15)
    # far left, silu(x) = x e^x (1 - e^x + ...): relative check against the limit
    assert abs(g[0, 0, -1, 0] / (-40.0 * math.exp(-40.0)) - 1.0) < 1e-12
    assert g[0, 0, 0, 0] == 0.0                        # silu(0) = 0 exactly
    assert np.all(th == 0.0)


def test_lowrank_bias_only():
    zg, zt, Ug, bg, Ut, bt = _factors(4)
    g, th = oracle.lowrank_gate_logits(zg, zt, np.zeros_like(Ug), bg, np.zeros_like(Ut), bt)
    assert np.array_equal(g, np.broadcast_to(bg[None, :, None, :], g.shape))
    assert np.array_equal(th, np.broadcast_to(bt[None, :, None, :], th.shape))
    # zero factor rows: silu(0) = 0, so the logits are the biases as well
    g0, th0 = oracle.lowrank_gate_logits(np.zeros_like(zg), np.zeros_like(zt), Ug, bg, Ut, bt)
    assert np.array_equal(g0, g) and np.array_equal(th0, th)


def test_lowrank_symmetries():
    zg, zt, Ug, bg, Ut, bt = _factors(5, B=2, H=4, T=6, dk=3, R=5)
    g, th = oracle.lowrank_gate_logits(zg, zt, Ug, bg, Ut, bt)
    # heads: permuting the per-head factors permutes the output heads
    perm = np.array([2, 0, 3, 1])
    gp, tp = oracle.lowrank_gate_logits(zg, zt, Ug[perm], bg[perm], Ut[perm], bt[perm])
    assert np.allclose(gp, g[:, perm]) and np.allclose(tp, th[:, perm])
    # tokens and batches: each token's logits depend on its own factor rows only
    gr, trr = oracle.lowrank_gate_logits(zg[::-1, ::-1], zt[::-1, ::-1], Ug, bg, Ut, bt)
    assert np.allclose(gr, g[::-1, :, ::-1]) and np.allclose(trr, th[::-1, :, ::-1])
    # ranks: the order of the rank index does not matter, and the rank sum splits
    rp = np.array([4, 2, 0, 1, 3])
    gq, tq = oracle.lowrank_gate_logits(zg[..., rp], zt[..., rp], Ug[..., rp], bg, Ut[..., rp], bt)
    assert np.allclose(gq, g) and np.allclose(tq, th)
    g1, t1 = oracle.lowrank_gate_logits(zg[..., :2], zt[..., :2], Ug[..., :2], bg, Ut[..., :2], bt)
    g2, t2 = oracle.lowrank_gate_logits(zg[..., 2:], zt[..., 2:], Ug[..., 2:], np.zeros_like(bg), Ut[..., 2:],
                                        np.zeros_like(bt))
    assert np.allclose(g1 + g2, g) and np.allclose(t1 + t2, th)
    # the temperature logits are linear in their factor rows (no activation)
    t2x = oracle.lowrank_gate_logits(zg, 2.0 * zt, Ug, bg, Ut, np.zeros_like(bt))[1]
    t1x = oracle.lowrank_gate_logits(zg, zt, Ug, bg, Ut, np.zeros_like(bt))[1]
    assert np.allclose(t2x, 2.0 * t1x)


@pytest.mark.parametrize("gbias,tbias", [(0.7, 0.3), (-1.2, 1.5), (2.0, -0.5)])
def test_lowrank_scan_geometric_closed_form(gbias, tbias):
    """Factor weights zero, biases constant: every token has the same gates,
    a = sigmoid(b_g)^sigmoid(b_tau) and beta = (1 - sigmoid(b_g))^sigmoid(b_tau)
    (the power form of the gate map), and with q_t = k_t = e_i, v_t = 1 the
    output of channel i is the geometric sum beta (1 - a^{t+1}) / (1 - a)."""
    B, H, T, dk, dv, R = 1, 2, 40, 4, 3, 4
    rng = np.random.default_rng(6)
    zg = rng.standard_normal((B, T, R))
    zt = rng.standard_normal((B, T, R))
    Ug = np.zeros((H, dk, R))
    Ut = np.zeros((H, dk, R))
    bg = np.full((H, dk), gbias)
    bt = np.full((H, dk), tbias)
    i = 2
    q = np.zeros((B, H, T, dk))
    q[..., i] = 1.0
    k = q.copy()
    v = np.ones((B, H, T, dv))
    o, _ = oracle.scan_lowrank(q, k, v, zg, zt, Ug, bg, Ut, bt)
    s, tau = expit(gbias), expit(tbias)
    a, beta = s ** tau, (1.0 - s) ** tau
    t = np.arange(T)
    ref = beta * (1.0 - a ** (t + 1)) / (1.0 - a)
    assert np.allclose(o[0, :, :, 0], ref[None, :], rtol=1e-12)
    assert np.allclose(o[0, :, :, 2], ref[None, :], rtol=1e-12)


def test_lowrank_scan_equals_scan_on_the_logits():
    rng = np.random.default_rng(7)
    B, H, T, dk, dv, R = 1, 2, 12, 4, 3, 5
    zg, zt, Ug, bg, Ut, bt = _factors(8, B, H, T, dk, R)
    q, k = rng.standard_normal((2, B, H, T, dk)) * 0.5
    v = rng.standard_normal((B, H, T, dv))
    act = zg * expit(zg)
    g = np.einsum("btr,hcr->bhtc", act, Ug) + bg[None, :, None, :]
    th = np.einsum("btr,hcr->bhtc", zt, Ut) + bt[None, :, None, :]
    o1, s1 = oracle.scan_lowrank(q, k, v, zg, zt, Ug, bg, Ut, bt)
    o2, s2 = oracle.scan(q, k, v, g, th)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14) and np.allclose(s1, s2, rtol=1e-12, atol=1e-14)
