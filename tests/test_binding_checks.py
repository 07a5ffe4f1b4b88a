"""The Python binding rejects caller-supplied tensors that do not match what the
kernels will write or read (device, dtype, exact shape, contiguity), before any
library call: a CPU tensor's host pointer or an undersized buffer must never
reach a kernel."""
import pytest
import torch

import causal_self_attention_mha_amd as na

GPU = torch.device("cuda:0")


def test_check_buf_rejects_wrong_device_dtype_shape_layout():
    good = torch.empty((2, 3, 4), dtype=torch.float32)
    na._check_buf("x", good, torch.float32, (2, 3, 4), good.device)  # accepted
    with pytest.raises(ValueError, match="is on cpu"):
        na._check_buf("lse", good, torch.float32, (2, 3, 4), GPU)
    with pytest.raises(ValueError, match="dtype"):
        na._check_buf("lse", good.to(torch.bfloat16), torch.float32, (2, 3, 4), good.device)
    with pytest.raises(ValueError, match="shape"):
        na._check_buf("delta", good[:, :, :3], torch.float32, (2, 3, 4), good.device)
    with pytest.raises(ValueError, match="contiguous"):
        t = torch.empty((2, 4, 3), dtype=torch.float32).transpose(1, 2)
        na._check_buf("o", t, torch.float32, (2, 3, 4), good.device)


def test_check_workspace_size_device_layout():
    ws = torch.empty(100, dtype=torch.uint8)
    assert na._check_workspace(ws, 100, ws.device) == 100
    assert na._check_workspace(ws.view(torch.int32), 64, ws.device) == 100
    with pytest.raises(ValueError, match="needs 101"):
        na._check_workspace(ws, 101, ws.device)
    with pytest.raises(ValueError, match="is on cpu"):
        na._check_workspace(ws, 10, GPU)
    with pytest.raises(ValueError, match="contiguous"):
        na._check_workspace(torch.empty((10, 10), dtype=torch.uint8).t(), 10, ws.device)


@pytest.mark.gpu
def test_outputs_checked_before_any_call(dev):
    """CPU lse, a short delta, a bf16 lse, an undersized workspace, a CPU decode
    output: each raises ValueError and launches nothing."""
    B, T, H, D = 1, 64, 2, 128
    q = torch.randn((B, T, H, D), device=dev).to(torch.bfloat16)
    k, v, o, do = (torch.randn_like(q) for _ in range(4))
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="lse is on cpu"):
        na.attn_fwd(q, k, v, lse=torch.empty((B, H, T), dtype=torch.float32))
    with pytest.raises(ValueError, match="lse has dtype"):
        na.attn_fwd(q, k, v, lse=torch.empty((B, H, T), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="delta has shape"):
        na.attn_bwd(q, k, v, o, do, lse,
                    delta=torch.empty((B, H, T - 1), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError, match="lse is on cpu"):
        na.attn_bwd(q, k, v, o, do, lse.cpu())
    with pytest.raises(ValueError, match="workspace has"):
        na.attn_bwd(q, k, v, o, do, lse, workspace=torch.empty(16, dtype=torch.uint8, device=dev))
    qd = torch.randn((B, H, D), device=dev).to(torch.bfloat16)
    kc = torch.randn((B, 32, H, D), device=dev).to(torch.bfloat16)
    lens = torch.full((B,), 32, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="o is on cpu"):
        na.attn_decode(qd, kc, kc, lens, o=torch.empty((B, H, D), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse has shape"):
        na.attn_decode(qd, kc, kc, lens, lse=torch.empty((B, H + 1), dtype=torch.float32,
                                                        device=dev))
    with pytest.raises(ValueError, match="workspace has"):
        na.attn_decode(qd, kc, kc, lens, workspace=torch.empty(8, dtype=torch.uint8, device=dev))
    # the forward with the queries' prologue folded in: tables and rotated outputs
    cos = torch.zeros((T, D // 2), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="cos must be contiguous"):
        na.attn_fwd(q, k, v, rope=(cos.cpu(), cos))
    with pytest.raises(ValueError, match="T_tab >= T"):
        na.attn_fwd(q, k, v, rope=(cos[:T - 1], cos[:T - 1]))
    with pytest.raises(ValueError, match="q_rot has shape"):
        na.attn_fwd(q, k, v, rope=(cos, cos), q_rot=torch.empty_like(q)[:, :T - 1])
    with pytest.raises(ValueError, match="k_rot is on cpu"):
        na.attn_fwd(q, k, v, rope=(cos, cos), k_rot=torch.empty(k.shape, dtype=k.dtype))
    torch.cuda.synchronize()
