"""Thin Python binding of librodimus.so (the MI355X Rodimus* token-mixer kernels).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/rodimus.h``.  PyTorch supplies
device memory and the current HIP stream; nothing here computes.

Entry points (same names as the C ABI):

* :func:`rodimus_scan_prefill` -- chunkwise-parallel prefill of the DDTS-gated
  recurrence; returns ``(o, S_T)``.
* :func:`rodimus_scan_prefill_lowrank` -- the prefill with the gate logits
  expanded inside the kernels from rank-16 factor rows; returns ``(o, S_T)``.
* :func:`rodimus_scan_prefill_noalloc` -- the same prefill into caller-given
  outputs, with its scratch in the library's fixed device array: allocates
  nothing, here or in the library.
* :func:`rodimus_scan_backward` -- gradients of the prefill with respect to q, k,
  v, g, tau and S0 (fp32); returns a dict.
* :func:`rodimus_decode_step`  -- one recurrent step on a resident state
  (in place by default); returns ``o``.
* :func:`sw_ska_attn`          -- sliding-window shared-key attention; returns ``o``.
* :func:`sw_ska_decode_step`   -- one SW-SKA token per sequence over ring-buffer
  window caches (appends the token, advances ``pos``); returns ``o``.

Every tensor's shape is checked against the others before the call, since the
C ABI receives bare pointers.

If the shared library has not been built, importing works but every call
raises ``RuntimeError``; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librodimus.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_TOO_LARGE = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
EXPORTED = ("rodimus_scan_prefill_workspace_bytes", "rodimus_scan_prefill", "rodimus_scan_prefill_noalloc",
            "rodimus_scan_prefill_lowrank",
            "rodimus_scan_prefill_varlen_workspace_bytes", "rodimus_scan_prefill_varlen",
            "rodimus_scan_backward_workspace_bytes", "rodimus_scan_backward",
            "rodimus_scan_backward_varlen_workspace_bytes", "rodimus_scan_backward_varlen", "rodimus_decode_step",
            "sw_ska_attn", "sw_ska_decode_workspace_bytes", "sw_ska_decode_step",
            "rodimus_status_string")

_lib = None


class RodimusError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gated_linear_attention_ddts_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.rodimus_scan_prefill_workspace_bytes.argtypes = [i] * 7
        L.rodimus_scan_prefill_workspace_bytes.restype = sz
        L.rodimus_scan_prefill.argtypes = [vp] * 8 + [i] * 7 + [vp, sz, vp]
        L.rodimus_scan_prefill.restype = i
        L.rodimus_scan_prefill_noalloc.argtypes = [vp] * 8 + [i] * 7 + [vp]
        L.rodimus_scan_prefill_noalloc.restype = i
        L.rodimus_scan_prefill_lowrank.argtypes = [vp] * 12 + [i] * 8 + [vp, sz, vp]
        L.rodimus_scan_prefill_lowrank.restype = i
        L.rodimus_scan_prefill_varlen_workspace_bytes.argtypes = [i] * 7
        L.rodimus_scan_prefill_varlen_workspace_bytes.restype = sz
        L.rodimus_scan_prefill_varlen.argtypes = [vp] * 9 + [i] * 8 + [vp, sz, vp]
        L.rodimus_scan_prefill_varlen.restype = i
        L.rodimus_scan_backward_workspace_bytes.argtypes = [i] * 6
        L.rodimus_scan_backward_workspace_bytes.restype = sz
        L.rodimus_scan_backward.argtypes = [vp] * 14 + [i] * 6 + [vp, sz, vp]
        L.rodimus_scan_backward.restype = i
        L.rodimus_scan_backward_varlen_workspace_bytes.argtypes = [i] * 6
        L.rodimus_scan_backward_varlen_workspace_bytes.restype = sz
        L.rodimus_scan_backward_varlen.argtypes = [vp] * 15 + [i] * 7 + [vp, sz, vp]
        L.rodimus_scan_backward_varlen.restype = i
        L.rodimus_decode_step.argtypes = [vp] * 8 + [i] * 5 + [vp]
        L.rodimus_decode_step.restype = i
        L.sw_ska_attn.argtypes = [vp] * 4 + [i] * 6 + [ctypes.c_float, i, vp]
        L.sw_ska_attn.restype = i
        L.sw_ska_decode_workspace_bytes.argtypes = [i] * 6
        L.sw_ska_decode_workspace_bytes.restype = sz
        L.sw_ska_decode_step.argtypes = [vp] * 7 + [i] * 5 + [ctypes.c_float, i, vp, sz, vp]
        L.sw_ska_decode_step.restype = i
        L.rodimus_status_string.argtypes = [i]
        L.rodimus_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().rodimus_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if t.get_device() != torch.cuda.current_device():
        raise ValueError("tensors must be on the current device (torch.cuda.set_device)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _out_dtype(t: Optional[torch.Tensor], dtype, name: str):
    """A caller-supplied output must have the dtype the kernel writes (a
    narrower one would be written past its end)."""
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _shape(t: Optional[torch.Tensor], shape, name: str):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != OK:
        raise RodimusError(status, where)


def rodimus_scan_prefill_workspace_bytes(B, H, T, dk, dv, chunk=64, dtype=BF16) -> int:
    return int(lib().rodimus_scan_prefill_workspace_bytes(B, H, T, dk, dv, chunk, dtype))


def rodimus_scan_prefill(q, k, v, g, tau, S0=None, chunk: int = 64, *, o=None, S_T=None,
                         want_state: bool = True, workspace=None,
                         stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q, k, g, tau: [B,H,T,dk]; v: [B,H,T,dv]; S0: [B,H,dk,dv] float32 or None.
    Returns (o [B,H,T,dv], S_T [B,H,dk,dv] float32 or None)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    for x in (k, g, tau, v):
        if x.dtype != q.dtype:
            raise TypeError("q, k, v, g, tau must share one dtype")
    for x, nm in ((k, "k"), (g, "g"), (tau, "tau")):
        _shape(x, (B, H, T, dk), nm)
    _shape(v, (B, H, T, dv), "v")
    _shape(S0, (B, H, dk, dv), "S0")
    _shape(o, (B, H, T, dv), "o")
    _shape(S_T, (B, H, dk, dv), "S_T")
    for x, nm in ((S0, "S0"), (S_T, "S_T")):
        if x is not None and x.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    _out_dtype(o, q.dtype, "o")
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    need = rodimus_scan_prefill_workspace_bytes(B, H, T, dk, dv, chunk, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().rodimus_scan_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(tau), _ptr(S0),
                                    _ptr(o), _ptr(S_T), B, H, T, dk, dv, chunk, dt,
                                    _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "rodimus_scan_prefill")
    return o, S_T


def rodimus_scan_prefill_lowrank(q, k, v, zg, zt, Ug, bg, Ut, bt, S0=None, chunk: int = 64, *, o=None,
                                 S_T=None, want_state: bool = True, workspace=None,
                                 stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q, k: [B,H,T,dk]; v: [B,H,T,dv] (bf16); zg, zt: [B,T,R] bf16 factor rows
    shared by the heads; Ug, Ut: [H,dk,R] bf16; bg, bt: [H,dk] float32.
    Per head: g = silu(zg) Ug^T + bg, tau = zt Ut^T + bt, then the prefill.
    Returns (o [B,H,T,dv], S_T [B,H,dk,dv] float32 or None)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    R = zg.shape[-1]
    dt = _dtype_code(q)
    for x in (k, v, zg, zt, Ug, Ut):
        if x.dtype != q.dtype:
            raise TypeError("q, k, v, zg, zt, Ug, Ut must share one dtype")
    _shape(k, (B, H, T, dk), "k")
    _shape(v, (B, H, T, dv), "v")
    _shape(zg, (B, T, R), "zg")
    _shape(zt, (B, T, R), "zt")
    _shape(Ug, (H, dk, R), "Ug")
    _shape(Ut, (H, dk, R), "Ut")
    _shape(bg, (H, dk), "bg")
    _shape(bt, (H, dk), "bt")
    _shape(S0, (B, H, dk, dv), "S0")
    _shape(o, (B, H, T, dv), "o")
    _shape(S_T, (B, H, dk, dv), "S_T")
    for x, nm in ((bg, "bg"), (bt, "bt"), (S0, "S0"), (S_T, "S_T")):
        if x is not None and x.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    _out_dtype(o, q.dtype, "o")
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    need = rodimus_scan_prefill_workspace_bytes(B, H, T, dk, dv, chunk, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().rodimus_scan_prefill_lowrank(_ptr(q), _ptr(k), _ptr(v), _ptr(zg), _ptr(zt), _ptr(Ug), _ptr(bg),
                                            _ptr(Ut), _ptr(bt), _ptr(S0), _ptr(o), _ptr(S_T), B, H, T, dk, dv, R,
                                            chunk, dt, _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "rodimus_scan_prefill_lowrank")
    return o, S_T


def rodimus_scan_prefill_noalloc(q, k, v, g, tau, S0=None, chunk: int = 64, *, o, S_T=None,
                                 stream=None) -> None:
    """rodimus_scan_prefill into the caller's o [B,H,T,dv] (and S_T
    [B,H,dk,dv] float32, or None to skip it), without any allocation: the
    segment states live in the library's fixed per-GPU scratch array.  Calls
    that may overlap on one GPU must be serialised by the caller."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    for x in (k, g, tau, v):
        if x.dtype != q.dtype:
            raise TypeError("q, k, v, g, tau must share one dtype")
    for x, nm in ((k, "k"), (g, "g"), (tau, "tau")):
        _shape(x, (B, H, T, dk), nm)
    _shape(v, (B, H, T, dv), "v")
    _shape(S0, (B, H, dk, dv), "S0")
    _shape(o, (B, H, T, dv), "o")
    _shape(S_T, (B, H, dk, dv), "S_T")
    for x, nm in ((S0, "S0"), (S_T, "S_T")):
        if x is not None and x.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    _out_dtype(o, q.dtype, "o")
    st = lib().rodimus_scan_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(tau), _ptr(S0),
                                            _ptr(o), _ptr(S_T), B, H, T, dk, dv, chunk, dt, _stream(stream))
    _check(st, "rodimus_scan_prefill_noalloc")


def rodimus_scan_prefill_varlen_workspace_bytes(N, H, max_seqlen, dk, dv, chunk=64, dtype=BF16) -> int:
    return int(lib().rodimus_scan_prefill_varlen_workspace_bytes(N, H, max_seqlen, dk, dv, chunk, dtype))


def rodimus_scan_prefill_varlen(q, k, v, g, tau, cu_seqlens, max_seqlen: int, S0=None, chunk: int = 64, *,
                                o=None, S_T=None, want_state: bool = True, workspace=None,
                                stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Packed ragged batch.  q, k, g, tau: [H,total,dk]; v: [H,total,dv];
    cu_seqlens: int32 [N+1] on the device (sequence s = rows cu[s]..cu[s+1]-1);
    max_seqlen >= every length; S0: [N,H,dk,dv] float32 or None.
    Returns (o [H,total,dv], S_T [N,H,dk,dv] float32 or None)."""
    H, total, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise TypeError("cu_seqlens must be a contiguous 1-D int32 tensor")
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs N + 1 >= 1 entries")
    for x in (k, g, tau, v):
        if x.dtype != q.dtype:
            raise TypeError("q, k, v, g, tau must share one dtype")
    for x, nm in ((k, "k"), (g, "g"), (tau, "tau")):
        _shape(x, (H, total, dk), nm)
    _shape(v, (H, total, dv), "v")
    _shape(S0, (N, H, dk, dv), "S0")
    _shape(o, (H, total, dv), "o")
    _shape(S_T, (N, H, dk, dv), "S_T")
    for x, nm in ((S0, "S0"), (S_T, "S_T")):
        if x is not None and x.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    _out_dtype(o, q.dtype, "o")
    if o is None:
        o = torch.empty((H, total, dv), dtype=q.dtype, device=q.device)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    need = rodimus_scan_prefill_varlen_workspace_bytes(N, H, max_seqlen, dk, dv, chunk, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().rodimus_scan_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(tau), _ptr(S0),
                                           _ptr(o), _ptr(S_T), _ptr(cu_seqlens), N, H, total, max_seqlen,
                                           dk, dv, chunk, dt, _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "rodimus_scan_prefill_varlen")
    return o, S_T


def rodimus_scan_backward_workspace_bytes(B, H, T, dk, dv, dtype=BF16) -> int:
    return int(lib().rodimus_scan_backward_workspace_bytes(B, H, T, dk, dv, dtype))


def rodimus_scan_backward(q, k, v, g, tau, dO, S0=None, dS_T=None, *, want_dS0: bool = True,
                          workspace=None, stream=None) -> dict:
    """Gradients of sum(dO * o) + sum(dS_T * S_T) of rodimus_scan_prefill with
    respect to q, k, v, g, tau (shaped like them) and S0 ([B,H,dk,dv]), all
    float32.  Returns dict(dq, dk, dv, dg, dtau, dS0)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    for x, nm in ((k, "k"), (g, "g"), (tau, "tau")):
        _shape(x, (B, H, T, dk), nm)
    _shape(v, (B, H, T, dv), "v")
    _shape(dO, (B, H, T, dv), "dO")
    _shape(S0, (B, H, dk, dv), "S0")
    _shape(dS_T, (B, H, dk, dv), "dS_T")
    for x in (k, g, tau, v, dO):
        if x.dtype != q.dtype:
            raise TypeError("q, k, v, g, tau, dO must share one dtype")
    for x, nm in ((S0, "S0"), (dS_T, "dS_T")):
        if x is not None and x.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    f32 = dict(dtype=torch.float32, device=q.device)
    out = dict(dq=torch.empty((B, H, T, dk), **f32), dk=torch.empty((B, H, T, dk), **f32),
               dv=torch.empty((B, H, T, dv), **f32), dg=torch.empty((B, H, T, dk), **f32),
               dtau=torch.empty((B, H, T, dk), **f32),
               dS0=torch.empty((B, H, dk, dv), **f32) if want_dS0 else None)
    need = rodimus_scan_backward_workspace_bytes(B, H, T, dk, dv, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().rodimus_scan_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(tau), _ptr(S0), _ptr(dO),
                                     _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                     _ptr(out["dg"]), _ptr(out["dtau"]), _ptr(out["dS0"]), B, H, T, dk,
                                     dv, dt, _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "rodimus_scan_backward")
    return out


def rodimus_scan_backward_varlen_workspace_bytes(N, H, max_seqlen, dk, dv, dtype=BF16) -> int:
    return int(lib().rodimus_scan_backward_varlen_workspace_bytes(N, H, max_seqlen, dk, dv, dtype))


def rodimus_scan_backward_varlen(q, k, v, g, tau, dO, cu_seqlens, max_seqlen: int, S0=None, dS_T=None, *,
                                 want_dS0: bool = True, out: Optional[dict] = None, workspace=None,
                                 stream=None) -> dict:
    """Backward of rodimus_scan_prefill_varlen over the same packed batch.
    q, k, g, tau: [H,total,dk]; v, dO: [H,total,dv]; cu_seqlens: int32 [N+1]
    on the device; S0, dS_T: [N,H,dk,dv] float32 or None.  Returns dict(dq,
    dk, dv, dg, dtau) shaped like the inputs and dS0 [N,H,dk,dv], all float32;
    `out` may supply those tensors (rows no sequence covers stay untouched)."""
    H, total, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise TypeError("cu_seqlens must be a contiguous 1-D int32 tensor")
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs N + 1 >= 1 entries")
    for x in (k, g, tau, v, dO):
        if x.dtype != q.dtype:
            raise TypeError("q, k, v, g, tau, dO must share one dtype")
    for x, nm in ((k, "k"), (g, "g"), (tau, "tau")):
        _shape(x, (H, total, dk), nm)
    _shape(v, (H, total, dv), "v")
    _shape(dO, (H, total, dv), "dO")
    _shape(S0, (N, H, dk, dv), "S0")
    _shape(dS_T, (N, H, dk, dv), "dS_T")
    for x, nm in ((S0, "S0"), (dS_T, "dS_T")):
        if x is not None and x.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    f32 = dict(dtype=torch.float32, device=q.device)
    shapes = dict(dq=(H, total, dk), dk=(H, total, dk), dv=(H, total, dv), dg=(H, total, dk),
                  dtau=(H, total, dk), dS0=(N, H, dk, dv))
    out = dict(out or {})
    for nm, shp in shapes.items():
        if out.get(nm) is None:
            if nm != "dS0" or want_dS0:
                out[nm] = torch.empty(shp, **f32)
            else:
                out[nm] = None
        else:
            _shape(out[nm], shp, nm)
            if out[nm].dtype != torch.float32:
                raise TypeError(f"{nm} must be float32")
    need = rodimus_scan_backward_varlen_workspace_bytes(N, H, max_seqlen, dk, dv, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().rodimus_scan_backward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(tau), _ptr(S0), _ptr(dO),
                                            _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                            _ptr(out["dg"]), _ptr(out["dtau"]), _ptr(out["dS0"]),
                                            _ptr(cu_seqlens), N, H, total, max_seqlen, dk, dv, dt,
                                            _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "rodimus_scan_backward_varlen")
    return out


def rodimus_decode_step(q, k, v, g, tau, S_in, S_out=None, *, o=None, stream=None) -> torch.Tensor:
    """q, k, g, tau: [N,H,dk]; v: [N,H,dv]; S_in: [N,H,dk,dv] float32.
    S_out defaults to S_in (update in place).  Returns o [N,H,dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    if S_out is None:
        S_out = S_in
    for x, nm in ((k, "k"), (g, "g"), (tau, "tau")):
        _shape(x, (N, H, dk), nm)
    _shape(v, (N, H, dv), "v")
    for x in (k, v, g, tau):
        if x.dtype != q.dtype:
            raise TypeError("q, k, v, g, tau must share one dtype")
    _shape(S_in, (N, H, dk, dv), "S_in")
    _shape(S_out, (N, H, dk, dv), "S_out")
    _shape(o, (N, H, dv), "o")
    if S_in.dtype != torch.float32 or S_out.dtype != torch.float32:
        raise TypeError("the state must be float32")
    _out_dtype(o, q.dtype, "o")
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    st = lib().rodimus_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(tau), _ptr(S_in),
                                   _ptr(S_out), _ptr(o), N, H, dk, dv, dt, _stream(stream))
    _check(st, "rodimus_decode_step")
    return o


def sw_ska_attn(q, k_shared, v, window: int, scale: Optional[float] = None, *, o=None,
                stream=None) -> torch.Tensor:
    """q: [B,H,T,dk]; k_shared: [B,T,dk]; v: [B,H,T,dv].  Returns o [B,H,T,dv]."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    _shape(k_shared, (B, T, dk), "k_shared")
    _shape(v, (B, H, T, dv), "v")
    _shape(o, (B, H, T, dv), "o")
    if k_shared.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k_shared, v must share one dtype")
    _out_dtype(o, q.dtype, "o")
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    st = lib().sw_ska_attn(_ptr(q), _ptr(k_shared), _ptr(v), _ptr(o), B, H, T, dk, dv, int(window),
                           float(scale), dt, _stream(stream))
    _check(st, "sw_ska_attn")
    return o


def sw_ska_decode_workspace_bytes(N, H, dk, dv, window, dtype=BF16) -> int:
    return int(lib().sw_ska_decode_workspace_bytes(N, H, dk, dv, window, dtype))


def sw_ska_decode_step(q, k_new, v_new, k_cache, v_cache, pos, scale: Optional[float] = None, *,
                       o=None, workspace=None, stream=None) -> torch.Tensor:
    """q: [N,H,dk]; k_new: [N,dk]; v_new: [N,H,dv]; k_cache: [N,W,dk];
    v_cache: [N,H,W,dv]; pos: [N] int32 (tokens seen; advanced by one).
    Writes the token into slot pos mod W of the caches.  Returns o [N,H,dv]."""
    N, H, dk = q.shape
    dv = v_new.shape[-1]
    W = k_cache.shape[1]
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    _shape(k_new, (N, dk), "k_new")
    _shape(v_new, (N, H, dv), "v_new")
    _shape(k_cache, (N, W, dk), "k_cache")
    _shape(v_cache, (N, H, W, dv), "v_cache")
    _shape(pos, (N,), "pos")
    _shape(o, (N, H, dv), "o")
    for x in (k_new, v_new, k_cache, v_cache):
        if x.dtype != q.dtype:
            raise TypeError("q, k_new, v_new and the caches must share one dtype")
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    _out_dtype(o, q.dtype, "o")
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    need = sw_ska_decode_workspace_bytes(N, H, dk, dv, W, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().sw_ska_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(pos), _ptr(o), N, H, dk, dv, W, float(scale), dt,
                                  _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "sw_ska_decode_step")
    return o
