"""Helpers for the GPU parity tests: move seeded host tensors to the device and
measure errors.  Error metric: err = max|x - r| / max|r| per output tensor."""
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
    den = np.max(np.abs(r))
    return float(np.max(np.abs(x - r)) / (den if den > 0 else 1.0))


# Tolerances from the stated bar: max relative error <= 2e-2 for bf16 inputs
# with an fp32 state, <= 1e-4 for the fp32 path.
TOL = {"bf16": 2e-2, "fp32": 1e-4}


def log(msg: str):
    print(msg, flush=True)
