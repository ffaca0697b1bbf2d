"""GPU parity of sw_ska_attn against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, dev, err, host, log

pytestmark = pytest.mark.gpu


def run(x, window, scale=None):
    d = {n: dev(x[n]) for n in ("q", "k", "v")}
    o = rd.sw_ska_attn(d["q"], d["k"], d["v"], window, scale)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("window", [1, 2, 17, 64, 100, 128, 129, 200, 10000])
def test_swska_windows(D, window):
    B, H, T = 1, 2, 300
    x = workloads.swska_inputs(31, B, H, T, D, D)
    log(f"swska D={D} w={window}")
    o = run(x, window)
    r = oracle.swska(x["q"].f64(), x["k"].f64(), x["v"].f64(), window)
    e = err(o, r)
    log(f"  err {e:.3e}")
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("B,H,T", [(2, 3, 131), (1, 16, 257), (1, 8, 64), (3, 1, 1), (1, 2, 5)])
def test_swska_batch_shapes(B, H, T):
    x = workloads.swska_inputs(32, B, H, T, 128, 128)
    o = run(x, 33)
    r = oracle.swska(x["q"].f64(), x["k"].f64(), x["v"].f64(), 33)
    assert err(o, r) <= TOL["bf16"]


def test_swska_peaked_scores():
    """q ~ N(0, 1) and k ~ N(0, 1): large score spread stresses the online max."""
    x = workloads.swska_inputs(33, 1, 2, 400, 128, 128, q_sigma=1.0, k_sigma=1.0)
    o = run(x, 150)
    r = oracle.swska(x["q"].f64(), x["k"].f64(), x["v"].f64(), 150)
    e = err(o, r)
    log(f"swska peaked err {e:.3e}")
    assert e <= TOL["bf16"]


def test_swska_custom_scale():
    x = workloads.swska_inputs(34, 1, 2, 160, 64, 64)
    o = run(x, 40, scale=0.3)
    r = oracle.swska(x["q"].f64(), x["k"].f64(), x["v"].f64(), 40, scale=0.3)
    assert err(o, r) <= TOL["bf16"]


def test_swska_window_one_is_v():
    x = workloads.swska_inputs(35, 1, 2, 150, 128, 128)
    o = run(x, 1)
    assert err(o, x["v"].f64()) <= 4e-3  # only the bf16 rounding of o


def test_swska_constant_key_is_window_mean():
    x = workloads.swska_inputs(36, 1, 2, 200, 128, 128)
    x["k"] = workloads.Tensor(np.repeat(x["k"].values[:, :1], 200, axis=1), "bf16")
    w = 37
    o = run(x, w)
    v = x["v"].f64()
    ref = np.stack([v[:, :, max(0, t - w + 1):t + 1].mean(axis=2) for t in range(200)], axis=2)
    assert err(o, ref) <= TOL["bf16"]


def test_swska_deterministic():
    x = workloads.swska_inputs(37, 1, 4, 333, 128, 128)
    assert np.array_equal(run(x, 77), run(x, 77))

