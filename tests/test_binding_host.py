"""The torch binding's argument checks, on the host: every bad tensor argument
is rejected with ValueError before any pointer reaches the library (no kernel
is launched in these tests; CPU tensors stand in for device ones, and the
binding only requires q to be on a GPU after every other check passed)."""
import pytest
import torch

import io_aware_exact_07_amd as fa

B, H, N, d = 2, 3, 40, 64


def qkv(dtype=torch.bfloat16):
    return [torch.zeros(B, H, N, d, dtype=dtype) for _ in range(5)]


def test_forward_rejects_a_bad_lse():
    q, k, v, _, _ = qkv()
    for bad in (torch.zeros(B, H, N, dtype=torch.bfloat16),        # wrong dtype
                torch.zeros(B, H, N - 1),                           # short
                torch.zeros(B, H, 2 * N)[..., ::2],                 # not contiguous
                torch.zeros(H, B, N)):                              # transposed shape
        with pytest.raises(ValueError, match="lse"):
            fa.forward(q, k, v, lse=bad)


def test_forward_rejects_a_bad_output():
    q, k, v, _, _ = qkv()
    with pytest.raises(ValueError, match="out"):
        fa.forward(q, k, v, out=torch.zeros(B, H, N, d))            # fp32 output for bf16 inputs


def test_forward_requires_device_tensors_last():
    q, k, v, _, _ = qkv()
    with pytest.raises(ValueError, match="GPU"):
        fa.forward(q, k, v, lse=torch.zeros(B, H, N))


def test_backward_rejects_a_bad_lse():
    q, k, v, o, do = qkv()
    for bad in (torch.zeros(B, H, N, dtype=torch.float64), torch.zeros(B, H, N + 1)):
        with pytest.raises(ValueError, match="lse"):
            fa.backward(q, k, v, o, do, bad)


def test_backward_rejects_a_short_workspace_counted_in_bytes():
    q, k, v, o, do = qkv()
    lse = torch.zeros(B, H, N)
    need = fa.fa_bwd_workspace_bytes(B, H, N, d, fa.FA_BF16)
    assert need > 0
    # float32 elements: need/4 elements hold exactly `need` bytes, one fewer does not
    with pytest.raises(ValueError, match="workspace"):
        fa.backward(q, k, v, o, do, lse, workspace=torch.zeros(need // 4 - 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        fa.backward(q, k, v, o, do, lse, workspace=torch.zeros(need // 4, dtype=torch.float32))


def test_backward_rejects_bad_gradient_buffers():
    q, k, v, o, do = qkv()
    lse = torch.zeros(B, H, N)
    with pytest.raises(ValueError, match="dq, dk, dv"):
        fa.backward(q, k, v, o, do, lse, grads=(torch.zeros_like(q), torch.zeros_like(q),
                                                torch.zeros(B, H, N, d)))
    with pytest.raises(ValueError, match="grads"):
        fa.backward(q, k, v, o, do, lse, grads=(torch.zeros_like(q),))


def test_seqlens_must_have_one_length_per_sequence():
    q, k, v, _, _ = qkv()
    with pytest.raises(ValueError, match="seqlens"):
        fa.forward(q, k, v, seqlens=torch.tensor([1, 2, 3]))
    q, k, v, o, do = qkv()
    with pytest.raises(ValueError, match="seqlens"):
        fa.backward(q, k, v, o, do, torch.zeros(B, H, N), seqlens=torch.tensor([4]))
