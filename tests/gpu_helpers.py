"""Helpers for the GPU parity tests: move seeded host tensors to the device and
measure errors.

Error metrics, per output tensor x against the oracle's r:
* err      = max|x - r| / max|r| over the whole tensor (the bar);
* per-(b,h) = the same ratio inside each (b,h) slice (the leading two axes, or
  whatever the caller says is one unit), worst slice reported, so that one head
  with small outputs cannot hide behind the others' scale;
* floored  = max over elements of |x - r| / max(|r|, 1e-3 max|r|), an
  element-wise relative error with a floor (near-zero outputs carry only an
  absolute error).
"""
import numpy as np
import torch

import workloads


def dev(t: "workloads.Tensor") -> torch.Tensor:
    """Device tensor in the storage dtype, bit-identical to the host values."""
    if t.dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(t.values)).cuda()
    bits = t.storage().view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(bits)).cuda().view(torch.bfloat16)


def host(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def err(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    assert np.all(np.isfinite(x)), "non-finite values in GPU output"
    den = np.max(np.abs(r)) if r.size else 0.0
    return float(np.max(np.abs(x - r)) / (den if den > 0 else 1.0)) if r.size else 0.0


def errs(x, r, unit_axes: int = 2) -> dict:
    """The three error figures above.  The first `unit_axes` axes index the
    independent units ((b,h) pairs, (n,h) pairs, sampled rows)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    g = err(x, r)
    nu = int(np.prod(r.shape[:unit_axes])) if unit_axes else 1
    xu = x.reshape(nu, -1)
    ru = r.reshape(nu, -1)
    den_u = np.max(np.abs(ru), axis=1)
    num_u = np.max(np.abs(xu - ru), axis=1)
    per_unit = np.where(den_u > 0, num_u / np.where(den_u > 0, den_u, 1.0), num_u)
    worst = int(np.argmax(per_unit))
    top = np.max(np.abs(r)) if r.size else 0.0
    floor = 1e-3 * top if top > 0 else 1.0
    floored = float(np.max(np.abs(x - r) / np.maximum(np.abs(r), floor))) if r.size else 0.0
    return {"err": g, "per_unit": float(per_unit[worst]), "worst_unit": worst, "floored": floored}


def fmt(name: str, e: dict) -> str:
    return (f"  {name}: err {e['err']:.3e}  worst unit {e['per_unit']:.3e} (#{e['worst_unit']})"
            f"  floored elementwise {e['floored']:.3e}")


# Tolerances from the stated bar: max relative error <= 2e-2 for bf16 inputs
# with an fp32 state, <= 1e-4 for the fp32 path.
TOL = {"bf16": 2e-2, "fp32": 1e-4}


def log(msg: str):
    print(msg, flush=True)
