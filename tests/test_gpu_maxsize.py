"""GPU parity at the largest sequence length each bf16 kernel accepts, where
the 32-bit buffer offsets (T * 256 bytes per tensor) are closest to their
limit.  Inputs are drawn on the device (workloads.device_normal); the oracle
reads back the exact bf16 values of the slices it checks.

* Prefill, T = 2^23 - 1 (131072 chunks of 64, a ragged last chunk, 256
  segments): a reset token 100 positions before the end (g = -40, tau = +40,
  so a ~ 4e-18 and beta ~ 1) makes the last 100 outputs and S_T depend only on
  those 100 tokens, so the oracle checks them exactly from S0 = 0.  The first
  100 outputs are checked from the start of the sequence.
* Backward, T = 2^23 - 1 (131072 checkpoint intervals, 256 segments): reset
  tokens at position 100 and 100 positions before the end.  The gradients of
  the first 100 tokens and dS0 then depend only on the first 100 tokens and
  their dO; those of the last 100 tokens only on the last 100.  The oracle's
  backward checks both slices exactly.
* SW-SKA, T = 2^23 - 1 at d = 128 (the largest T the entry point supports):
  rows sampled across the whole sequence, each computed by the oracle from its
  own window.
* SW-SKA decode at the largest window, 2^19 slots (2048 splits of 256): one
  sequence with a full, wrapped window whose new token lands in the very last
  slot, and one with 301 valid slots (2046 splits without any, which the
  combine must weigh as zero).  The oracle computes each head's row over the
  window gathered from the caches after the step.
"""
import numpy as np
import pytest
import torch

import gated_linear_attention_ddts_amd as rd
import oracle
import workloads
from tests.gpu_helpers import TOL, err, host, log

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "theta")
T_MAX = (1 << 23) - 1


def _scan_inputs_on_device(T, seed):
    s = 1.0 / np.sqrt(128)
    shp = (1, 1, T, 128)
    return dict(q=workloads.device_normal(shp, seed, 0.0, s), k=workloads.device_normal(shp, seed + 1, 0.0, s),
                v=workloads.device_normal(shp, seed + 2), g=workloads.device_normal(shp, seed + 3),
                theta=workloads.device_normal(shp, seed + 4))


def test_prefill_max_T_reset_tail():
    T, tail = T_MAX, 100
    log(f"prefill max T={T}: inputs on the device")
    d = _scan_inputs_on_device(T, 71)
    tr = T - tail
    d["g"][0, 0, tr].fill_(-40.0)
    d["theta"][0, 0, tr].fill_(40.0)
    log("prefill max T: GPU")
    o, ST = rd.rodimus_scan_prefill(*(d[n] for n in NAMES), None, 64)
    torch.cuda.synchronize()
    log("prefill max T: oracle on the head and the tail")
    head = [host(d[n][:, :, :tail]) for n in NAMES]
    ro, _ = oracle.scan(*head, nthreads=1)
    assert err(host(o[:, :, :tail]), ro) <= TOL["bf16"]
    tl = [host(d[n][:, :, tr:]) for n in NAMES]
    ro, rST = oracle.scan(*tl, nthreads=1)
    eo, es = err(host(o[:, :, tr:]), ro), err(host(ST), rST)
    log(f"  tail err o {eo:.3e}  S_T {es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    # every output finite, checked on the device in slices
    for c0 in range(0, T, 1 << 21):
        assert torch.isfinite(o[:, :, c0:c0 + (1 << 21)].float()).all()


def test_backward_max_T_reset_head_and_tail():
    T, n = T_MAX, 100
    log(f"backward max T={T}: inputs on the device")
    d = _scan_inputs_on_device(T, 91)
    dO = workloads.device_normal((1, 1, T, 128), 96)
    tr = T - n
    for p in (n, tr):
        d["g"][0, 0, p].fill_(-40.0)
        d["theta"][0, 0, p].fill_(40.0)
    log("backward max T: GPU")
    out = rd.rodimus_scan_backward(*(d[x] for x in NAMES), dO)
    torch.cuda.synchronize()
    log("backward max T: every gradient finite (on the device, in slices)")
    for kk in ("dq", "dk", "dv", "dg", "dtau"):
        for c0 in range(0, T, 1 << 21):
            assert torch.isfinite(out[kk][:, :, c0:c0 + (1 << 21)]).all(), kk
    assert torch.isfinite(out["dS0"]).all()
    log("backward max T: oracle on the head and the tail")
    for name, sl in (("head", slice(0, n)), ("tail", slice(tr, T))):
        ref = oracle.scan_backward(*(host(d[x][:, :, sl]) for x in NAMES), host(dO[:, :, sl]))
        ref["dtau"] = ref.pop("dtheta")
        errs = {kk: err(host(out[kk][:, :, sl]), ref[kk]) for kk in ("dq", "dk", "dv", "dg", "dtau")}
        if name == "head":
            errs["dS0"] = err(host(out["dS0"]), ref["dS0"])
        log(f"  {name}: " + " ".join(f"{k} {e:.2e}" for k, e in errs.items()))
        for kk, e in errs.items():
            assert e <= TOL["bf16"], (name, kk, e)


def test_swska_max_T_sampled_rows():
    T, w, H = T_MAX, 4096, 1
    log(f"swska max T={T}: inputs on the device")
    q = workloads.device_normal((1, H, T, 128), 81, 0.0, 1.0 / np.sqrt(128))
    k = workloads.device_normal((1, T, 128), 82)
    v = workloads.device_normal((1, H, T, 128), 83)
    log("swska max T: GPU")
    o = rd.sw_ska_attn(q, k, v, w)
    torch.cuda.synchronize()
    rows = [0, 1, 4095, 4096, 1 << 22, (1 << 23) - 4097, T - 2, T - 1]
    log(f"swska max T: oracle on rows {rows}")
    for t in rows:
        lo = max(0, t - w + 1)
        sl = slice(lo, t + 1)
        ro = oracle.swska(host(q[:, :, sl]), host(k[:, sl]), host(v[:, :, sl]), w, 1.0 / np.sqrt(128),
                          rows=[t - lo])
        e = err(host(o[:, :, t]), ro[:, :, t - lo])
        assert e <= TOL["bf16"], (t, e)


def test_swska_decode_max_window():
    N, H, d, W = 2, 2, 128, 1 << 19
    ts = [3 * W - 1, 300]
    log(f"swska decode max window W={W}: caches on the device")
    kc = workloads.device_normal((N, W, d), 91)
    vc = workloads.device_normal((N, H, W, d), 92)
    q = workloads.device_normal((N, H, d), 93, 0.0, 1.0 / np.sqrt(d))
    kn = workloads.device_normal((N, d), 94)
    vn = workloads.device_normal((N, H, d), 95)
    pos = torch.tensor(ts, dtype=torch.int32, device="cuda")
    o = rd.sw_ska_decode_step(q, kn, vn, kc, vc, pos)
    torch.cuda.synchronize()
    assert pos.cpu().tolist() == [t + 1 for t in ts]
    for n, t in enumerate(ts):
        log(f"swska decode max window: oracle for sequence {n} (t = {t})")
        ps = np.arange(max(0, t - W + 1), t + 1)
        slots = torch.from_numpy(ps % W).cuda()
        kw, vw = host(kc[n].index_select(0, slots)), host(vc[n].index_select(1, slots))
        L = len(ps)
        qs = np.zeros((1, H, L, d))
        qs[0, :, -1] = host(q[n])
        ref = oracle.swska(qs, kw[None], vw[None], W, rows=[h * L + L - 1 for h in range(H)], nthreads=8)
        e = err(host(o[n]), ref[0, :, -1])
        log(f"  err o {e:.3e}")
        assert e <= TOL["bf16"], (n, t, e)
        assert torch.equal(kc[n, t % W], kn[n]) and torch.equal(vc[n, :, t % W], vn[n])
