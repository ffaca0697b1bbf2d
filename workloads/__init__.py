"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws normal samples with
numpy's PCG64 generator and rounds them to the storage dtype.  Both the oracle
and the HIP path consume the values it returns.

Recipe (fixed, so that every consumer sees bit-identical inputs):

* ``rng = numpy.random.default_rng(seed)``;
* tensors are drawn in the order q, k, v, g, theta as fp64 N(mu, sigma^2) over the
  full C-order shape, then rounded to fp32 (round to nearest even) and, for bf16
  workloads, from fp32 to bf16 (round to nearest even);
* q, k ~ N(0, 1/dk); v ~ N(0, 1); g, theta ~ N(mu_gate, 1).

The shapes follow the Rodimus+ 1.6B module configuration (16 heads, head_dim
128, state expansion 2, window 4096, contexts up to 128K) given in section 3 of
the Rodimus* deployment blog (m.nxbn.cn/news/205411).  The pages' own evaluation
data (code/NLP suites, WikiText-103, MQAR, NeedleBench) is not available and is
not reproduced; these random tensors stand in for it.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def bf16_bits(x) -> np.ndarray:
    """Round to bf16 (nearest even, via fp32) and return the raw uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact fp32 value of bf16 bit patterns."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to(x, dtype: str) -> np.ndarray:
    """Round fp64 samples to the storage dtype and return them as exact fp32."""
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_to_f32(bf16_bits(x))
    raise ValueError(dtype)


@dataclass
class Tensor:
    """A host tensor: exact values (fp32) plus the storage dtype."""
    values: np.ndarray
    dtype: str

    @property
    def shape(self):
        return self.values.shape

    def f64(self) -> np.ndarray:
        return self.values.astype(np.float64)

    def storage(self) -> np.ndarray:
        """Array in the storage format: float32, or uint16 bf16 bits."""
        if self.dtype == "fp32":
            return self.values
        return bf16_bits(self.values)


def _draw(rng, shape, mu, sigma, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float64)
    if sigma != 1.0:
        x *= sigma
    if mu != 0.0:
        x += mu
    return Tensor(round_to(x, dtype), dtype)


def scan_inputs(seed, B, H, T, dk, dv, dtype="bf16", gate_mu=0.0, gate_sigma=1.0,
                qk_sigma=None, v_sigma=1.0):
    """q, k, v, g, theta for the prefill scan, drawn in that order."""
    rng = np.random.default_rng(seed)
    s = (1.0 / np.sqrt(dk)) if qk_sigma is None else qk_sigma
    q = _draw(rng, (B, H, T, dk), 0.0, s, dtype)
    k = _draw(rng, (B, H, T, dk), 0.0, s, dtype)
    v = _draw(rng, (B, H, T, dv), 0.0, v_sigma, dtype)
    g = _draw(rng, (B, H, T, dk), gate_mu, gate_sigma, dtype)
    th = _draw(rng, (B, H, T, dk), gate_mu, gate_sigma, dtype)
    return dict(q=q, k=k, v=v, g=g, theta=th)


def lowrank_inputs(seed, B, H, T, dk, dv, R=16, dtype="bf16", z_sigma=1.0, bias_sigma=0.5, gbias_mu=0.0,
                   tbias_mu=0.0):
    """Inputs of the prefill with low-rank gate factors, drawn in this order:
    q, k, v as scan_inputs (q, k ~ N(0, 1/dk), v ~ N(0, 1)); the factor rows
    zg, zt [B,T,R] ~ N(0, z_sigma^2); the per-head factors Ug, Ut [H,dk,R]
    ~ N(0, 1/R) (so each logit has about unit spread); all of those in the
    storage dtype; then the biases bg ~ N(gbias_mu, bias_sigma^2) and
    bt ~ N(tbias_mu, bias_sigma^2), [H,dk], fp32."""
    rng = np.random.default_rng(seed)
    s = 1.0 / np.sqrt(dk)
    q = _draw(rng, (B, H, T, dk), 0.0, s, dtype)
    k = _draw(rng, (B, H, T, dk), 0.0, s, dtype)
    v = _draw(rng, (B, H, T, dv), 0.0, 1.0, dtype)
    zg = _draw(rng, (B, T, R), 0.0, z_sigma, dtype)
    zt = _draw(rng, (B, T, R), 0.0, z_sigma, dtype)
    Ug = _draw(rng, (H, dk, R), 0.0, 1.0 / np.sqrt(R), dtype)
    Ut = _draw(rng, (H, dk, R), 0.0, 1.0 / np.sqrt(R), dtype)
    bg = _draw(rng, (H, dk), gbias_mu, bias_sigma, "fp32")
    bt = _draw(rng, (H, dk), tbias_mu, bias_sigma, "fp32")
    return dict(q=q, k=k, v=v, zg=zg, zt=zt, Ug=Ug, Ut=Ut, bg=bg, bt=bt)


def decode_pool(seed, N, H, dk, dv, pool=8, dtype="bf16", gate_mu=0.0):
    """``pool`` input sets for the decode step; step s uses set s mod pool."""
    rng = np.random.default_rng(seed)
    sets = []
    for _ in range(pool):
        q = _draw(rng, (N, H, dk), 0.0, 1.0 / np.sqrt(dk), dtype)
        k = _draw(rng, (N, H, dk), 0.0, 1.0 / np.sqrt(dk), dtype)
        v = _draw(rng, (N, H, dv), 0.0, 1.0, dtype)
        g = _draw(rng, (N, H, dk), gate_mu, 1.0, dtype)
        th = _draw(rng, (N, H, dk), gate_mu, 1.0, dtype)
        sets.append(dict(q=q, k=k, v=v, g=g, theta=th))
    return sets


def swska_inputs(seed, B, H, T, dk, dv, dtype="bf16", q_sigma=None, k_sigma=1.0, v_sigma=1.0):
    """q [B,H,T,dk], k_shared [B,T,dk], v [B,H,T,dv], drawn in that order."""
    rng = np.random.default_rng(seed)
    qs = (1.0 / np.sqrt(dk)) if q_sigma is None else q_sigma
    q = _draw(rng, (B, H, T, dk), 0.0, qs, dtype)
    k = _draw(rng, (B, T, dk), 0.0, k_sigma, dtype)
    v = _draw(rng, (B, H, T, dv), 0.0, v_sigma, dtype)
    return dict(q=q, k=k, v=v)


def device_normal(shape, seed, mu=0.0, sigma=1.0, dtype="bf16", device="cuda"):
    """N(mu, sigma^2) samples drawn on the device, for inputs too large to draw
    on the host (the maximum-length checks): torch's seeded Philox generator
    in fp32, then rounded to the storage dtype (nearest even).  Whoever needs
    exact values (the oracle) reads back the rounded tensor."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    if mu != 0.0:
        x.add_(mu)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def ragged_lengths(seed, N, total, min_len=1, sigma=0.8):
    """N sequence lengths that sum to `total` (each >= min_len): a seeded
    log-normal mix of short and long requests, as a dynamic batch packs them."""
    rng = np.random.default_rng(seed)
    w = rng.lognormal(0.0, sigma, size=N)
    extra = total - N * min_len
    if extra < 0:
        raise ValueError("total too small for N sequences of min_len")
    raw = w / w.sum() * extra
    L = np.floor(raw).astype(np.int64)
    # hand the rounding remainder to the largest fractional parts
    rem = int(extra - L.sum())
    L[np.argsort(raw - L)[::-1][:rem]] += 1
    return (L + min_len).astype(np.int64)


def cu_seqlens(lengths) -> np.ndarray:
    """Offsets [0, l0, l0+l1, ...] (int32) of a packed batch."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def packed_scan_inputs(seed, H, total, dk, dv, dtype="bf16"):
    """q, k, v, g, theta of a packed batch: [H, total, d] each, drawn as
    scan_inputs with B = 1 (the sequences' rows are independent draws)."""
    x = scan_inputs(seed, 1, H, total, dk, dv, dtype)
    return {n: Tensor(t.values[0], t.dtype) for n, t in x.items()}


# The workloads, named by what they are.
CONFIGS = {
    "tiny_fp32_scan": dict(kind="scan", B=1, H=2, T=256, dk=16, dv=32, dtype="fp32", chunk=32,
                           gate_mu=0.0, seed=1),
    "prefill_1p6b_T4096": dict(kind="scan", B=4, H=16, T=4096, dk=128, dv=128, dtype="bf16",
                               chunk=64, gate_mu=0.0, seed=2),
    "prefill_long_T131072": dict(kind="scan", B=1, H=16, T=131072, dk=128, dv=128, dtype="bf16",
                                 chunk=64, gate_mu=0.5, seed=3),
    "decode_N256": dict(kind="decode", N=256, H=16, dk=128, dv=128, dtype="bf16", steps=1000,
                        pool=8, seed=4),
    "swska_T32768_w4096": dict(kind="swska", B=1, H=16, T=32768, dk=128, dv=128, window=4096,
                               dtype="bf16", seed=5),
    # SW-SKA decode: 64 sequences whose 4096-slot window caches are full
    # (shared K [64, 4096, 128], per-head V [64, 16, 4096, 128]), one token per step
    "swska_decode_N64_w4096": dict(kind="swska_decode", N=64, H=16, dk=128, dv=128, window=4096,
                                   pos0=8192, steps=200, pool=8, dtype="bf16", seed=6),
    # a dynamic batch: 64 requests of log-normal lengths packed into 16384
    # tokens per head (the token count of the 1.6B batch), 16 heads
    "prefill_varlen_N64_16K": dict(kind="varlen", N=64, H=16, total=16384, min_len=16, dk=128,
                                   dv=128, dtype="bf16", chunk=64, seed=7),
    # the 1.6B-shaped prefill with the gate logits expanded in-kernel from
    # rank-16 factor rows shared by the heads (g and tau never stored); the
    # biases at their initial value 0 (b_tau = 0 is a temperature of 0.5, the
    # module's tempered_gate_init)
    "prefill_lowrank_1p6b_T4096": dict(kind="lowrank", B=4, H=16, T=4096, dk=128, dv=128, R=16,
                                       dtype="bf16", chunk=64, seed=9, bias_sigma=0.0),
}
