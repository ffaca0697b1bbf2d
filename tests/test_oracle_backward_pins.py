"""Pins of oracle.scan_backward against things other than itself (CPU only):

* central finite differences of the (separately pinned) forward oracle, for
  every element of every input, on tiny sizes;
* reverse-mode autograd of an independent plain recurrence written here in
  torch fp64 (its own gate map from torch.sigmoid / softplus);
* theta = -inf (a = beta = 1): the gradients of causal linear attention in
  closed form (numpy cumulative sums), and exactly zero gate gradients.
"""
import numpy as np
import pytest
import torch

import oracle

NAMES = ("q", "k", "v", "g", "theta")


def _inputs(seed, B=1, H=2, T=9, dk=3, dv=2, gate_mu=0.0):
    r = np.random.default_rng(seed)
    x = dict(q=r.standard_normal((B, H, T, dk)), k=r.standard_normal((B, H, T, dk)),
             v=r.standard_normal((B, H, T, dv)), g=r.standard_normal((B, H, T, dk)) + gate_mu,
             theta=r.standard_normal((B, H, T, dk)))
    S0 = r.standard_normal((B, H, dk, dv))
    dO = r.standard_normal((B, H, T, dv))
    dST = r.standard_normal((B, H, dk, dv))
    return x, S0, dO, dST


def _loss(x, S0, dO, dST):
    o, ST = oracle.scan(*(x[n] for n in NAMES), S0)
    return float(np.sum(dO * o) + (0.0 if dST is None else np.sum(dST * ST)))


@pytest.mark.parametrize("with_state", [False, True])
def test_backward_matches_central_differences(with_state):
    x, S0, dO, dST = _inputs(11 + with_state)
    if not with_state:
        S0, dST = None, None
    grads = oracle.scan_backward(*(x[n] for n in NAMES), dO, S0, dST)
    eps = 1e-6
    targets = [(n, x[n], "d" + n) for n in NAMES]
    if with_state:
        targets.append(("S0", S0, "dS0"))
    for name, arr, gname in targets:
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = arr[idx]
            arr[idx] = keep + eps
            lp = _loss(x, S0, dO, dST)
            arr[idx] = keep - eps
            lm = _loss(x, S0, dO, dST)
            arr[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grads[gname], num, rtol=1e-6, atol=1e-8, err_msg=name)


def _torch_reference(x, S0, dO, dST):
    """An independent plain recurrence in torch fp64, differentiated by autograd."""
    t = {n: torch.tensor(x[n], requires_grad=True) for n in NAMES}
    S0t = torch.tensor(S0, requires_grad=True)
    tau = torch.sigmoid(t["theta"])
    a = torch.exp(-tau * torch.nn.functional.softplus(-t["g"]))
    beta = torch.exp(-tau * torch.nn.functional.softplus(t["g"]))
    S = S0t
    outs = []
    T = x["q"].shape[2]
    for s in range(T):
        S = a[:, :, s, :, None] * S + (beta[:, :, s] * t["k"][:, :, s])[..., None] * t["v"][:, :, s, None, :]
        outs.append(torch.einsum("bhi,bhij->bhj", t["q"][:, :, s], S))
    o = torch.stack(outs, dim=2)
    loss = (torch.tensor(dO) * o).sum() + (torch.tensor(dST) * S).sum()
    loss.backward()
    res = {"d" + n: t[n].grad.numpy() for n in NAMES}
    res["dS0"] = S0t.grad.numpy()
    return res


def test_backward_matches_torch_autograd_of_a_plain_recurrence():
    x, S0, dO, dST = _inputs(21, B=2, H=2, T=33, dk=5, dv=4)
    ours = oracle.scan_backward(*(x[n] for n in NAMES), dO, S0, dST, nthreads=3)
    ref = _torch_reference(x, S0, dO, dST)
    for k in ref:
        np.testing.assert_allclose(ours[k], ref[k], rtol=1e-10, atol=1e-12, err_msg=k)


def test_backward_reduces_to_linear_attention_gradients():
    x, S0, dO, dST = _inputs(31, B=1, H=3, T=17, dk=4, dv=3)
    x["theta"][:] = -np.inf
    ours = oracle.scan_backward(*(x[n] for n in NAMES), dO, S0, dST)
    q, k, v = x["q"], x["k"], x["v"]
    # forward: S_t = S0 + sum_{s<=t} k_s^T v_s ;  o_t = q_t S_t
    S = S0[:, :, None] + np.cumsum(k[..., :, None] * v[..., None, :], axis=2)
    # G_t = dST + sum_{t'>=t} q_t'^T dO_t'  (reverse cumulative sum)
    qdo = q[..., :, None] * dO[..., None, :]
    G = dST[:, :, None] + np.flip(np.cumsum(np.flip(qdo, axis=2), axis=2), axis=2)
    np.testing.assert_allclose(ours["dq"], np.einsum("bhtj,bhtij->bhti", dO, S), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ours["dk"], np.einsum("bhtij,bhtj->bhti", G, v), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ours["dv"], np.einsum("bhti,bhtij->bhtj", k, G), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ours["dS0"], G[:, :, 0], rtol=1e-11, atol=1e-12)
    assert np.all(ours["dg"] == 0.0) and np.all(ours["dtheta"] == 0.0)


def test_backward_of_empty_sequence_passes_the_state_gradient():
    x, S0, dO, dST = _inputs(41, T=0)
    ours = oracle.scan_backward(*(x[n] for n in NAMES), dO, S0, dST)
    np.testing.assert_array_equal(ours["dS0"], dST)
