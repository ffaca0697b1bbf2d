"""Host-side checks of the Python binding: every tensor's shape and dtype is
validated before the C ABI receives bare pointers, so a mismatched output
buffer (which the kernel would write past its end) or a host tensor is refused
with an exception and nothing is launched.  Runs without a GPU."""
import pytest
import torch

import gated_linear_attention_ddts_amd as rd

bf16, f32 = torch.bfloat16, torch.float32


def _scan(B=1, H=2, T=8, dk=16, dv=32, dtype=bf16):
    mk = lambda *s: torch.zeros(*s, dtype=dtype)
    return mk(B, H, T, dk), mk(B, H, T, dk), mk(B, H, T, dv), mk(B, H, T, dk), mk(B, H, T, dk)


def test_prefill_rejects_an_output_of_another_dtype():
    q, k, v, g, tau = _scan(dtype=f32)
    with pytest.raises(TypeError, match="o must be"):
        rd.rodimus_scan_prefill(q, k, v, g, tau, o=torch.zeros(1, 2, 8, 32, dtype=bf16))
    with pytest.raises(TypeError, match="S_T must be float32"):
        rd.rodimus_scan_prefill(q, k, v, g, tau, S_T=torch.zeros(1, 2, 16, 32, dtype=bf16))


def test_prefill_rejects_mixed_input_dtypes_and_shapes():
    q, k, v, g, tau = _scan()
    with pytest.raises(TypeError):
        rd.rodimus_scan_prefill(q, k, v.float(), g, tau)
    with pytest.raises(ValueError, match="k has shape"):
        rd.rodimus_scan_prefill(q, k[:, :, :4], v, g, tau)


def test_varlen_prefill_rejects_an_output_of_another_dtype():
    H, total, d = 2, 10, 16
    x = [torch.zeros(H, total, d, dtype=f32) for _ in range(5)]
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(TypeError, match="o must be"):
        rd.rodimus_scan_prefill_varlen(*x, cu, 6, o=torch.zeros(H, total, d, dtype=bf16))
    with pytest.raises(TypeError, match="cu_seqlens"):
        rd.rodimus_scan_prefill_varlen(*x, cu.long(), 6)


def test_decode_checks_every_input_dtype_and_the_output():
    N, H, dk, dv = 2, 3, 16, 32
    q, k, g, tau = (torch.zeros(N, H, dk, dtype=f32) for _ in range(4))
    v = torch.zeros(N, H, dv, dtype=bf16)      # narrower than the fp32 the kernel would read
    S = torch.zeros(N, H, dk, dv, dtype=f32)
    with pytest.raises(TypeError, match="share one dtype"):
        rd.rodimus_decode_step(q, k, v, g, tau, S)
    with pytest.raises(TypeError, match="o must be"):
        rd.rodimus_decode_step(q, k, v.float(), g, tau, S, o=torch.zeros(N, H, dv, dtype=bf16))
    with pytest.raises(TypeError, match="state must be float32"):
        rd.rodimus_decode_step(q, k, v.float(), g, tau, S.double())


def test_swska_rejects_an_output_of_another_dtype():
    B, H, T, d = 1, 2, 5, 64
    q, v = torch.zeros(B, H, T, d, dtype=f32), torch.zeros(B, H, T, d, dtype=f32)
    k = torch.zeros(B, T, d, dtype=f32)
    with pytest.raises(TypeError, match="o must be"):
        rd.sw_ska_attn(q, k, v, 4, o=torch.zeros(B, H, T, d, dtype=bf16))


def test_swska_decode_rejects_an_output_of_another_dtype_and_a_wide_pos():
    N, H, W, d = 2, 3, 16, 64
    q, vn = torch.zeros(N, H, d, dtype=bf16), torch.zeros(N, H, d, dtype=bf16)
    kn, kc, vc = torch.zeros(N, d, dtype=bf16), torch.zeros(N, W, d, dtype=bf16), torch.zeros(N, H, W, d, dtype=bf16)
    pos = torch.zeros(N, dtype=torch.int32)
    with pytest.raises(TypeError, match="o must be"):
        rd.sw_ska_decode_step(q, kn, vn, kc, vc, pos, o=torch.zeros(N, H, d, dtype=f32))
    with pytest.raises(TypeError, match="pos must be int32"):
        rd.sw_ska_decode_step(q, kn, vn, kc, vc, pos.long())


def test_host_tensors_are_refused_before_any_launch():
    q, k, v, g, tau = _scan()
    with pytest.raises(ValueError, match="on the GPU"):
        rd.rodimus_scan_prefill(q, k, v, g, tau)
