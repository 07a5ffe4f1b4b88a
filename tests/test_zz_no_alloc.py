"""The decode entry point that allocates nothing (na_attn_decode_noalloc)
against na_attn_decode with a caller workspace: the same kernels, so the
outputs must agree bit for bit.  Two calls in a row on one device, the second
smaller than the first (the shared scratch keeps the first call's contents),
both through the C ABI."""
import ctypes

import numpy as np
import pytest

import workloads as W
from parity_util import to_device

pytestmark = pytest.mark.gpu


def _decode_both(na, dinp, dev):
    import torch
    lib = na.load_library()
    q, kc, vc = (to_device(x, dev) for x in (dinp.q_store, dinp.k_store, dinp.v_store))
    lens = torch.from_numpy(np.ascontiguousarray(dinp.seqlens)).to(dev)
    B, H, D = q.shape
    T_cap = kc.shape[1]
    o_ref, lse_ref = na.attn_decode(q, kc, vc, lens)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=dev)
    P = ctypes.c_void_p
    st = lib.na_attn_decode_noalloc(P(q.data_ptr()), P(kc.data_ptr()), P(vc.data_ptr()),
                                    P(lens.data_ptr()), P(o.data_ptr()), P(lse.data_ptr()), B, H, D,
                                    T_cap, P(torch.cuda.current_stream(dev).cuda_stream))
    assert st == 0, lib.na_last_error().decode()
    torch.cuda.synchronize()
    return o, lse, o_ref, lse_ref


def test_noalloc_decode_matches_workspace_decode(dev):
    import torch

    import causal_self_attention_mha_amd as na
    big = W.make_decode_inputs("decode_d20")  # B = 64, H = 10, T_cap = 2048: 11.0 MB of scratch
    small = W.make_decode_inputs(B=8, T_cap=700, H=4, seed=71)
    for dinp in (big, small):
        o, lse, o_ref, lse_ref = _decode_both(na, dinp, dev)
        assert torch.equal(o, o_ref)
        assert torch.equal(lse, lse_ref)
        assert bool(torch.isfinite(o.float()).all())
