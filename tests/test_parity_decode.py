"""GPU parity of the split-KV decode against the fp64 oracle, through the C
ABI.  The full d20 decode workload (64 sequences, 10 heads, lengths uniform
in [1, 2048]) is compared on every (b, h); cache rows at or beyond each
sequence's length are filled with NaN so that any read of them shows up."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import BF16_MAX_ABS, BF16_REL_L2, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def run_decode(inp, dev, poison=True, want_lse=True):
    import torch
    import causal_self_attention_mha_amd as na
    q = to_device(inp.q_store, dev)
    kc = to_device(inp.k_store, dev)
    vc = to_device(inp.v_store, dev)
    if poison:
        for b, L in enumerate(inp.seqlens):
            kc[b, int(L):] = float("nan")
            vc[b, int(L):] = float("nan")
    lens = torch.from_numpy(inp.seqlens.astype(np.int32)).to(dev)
    o, lse = na.attn_decode(q, kc, vc, lens, want_lse=want_lse)
    torch.cuda.synchronize()
    return o, lse


def check(inp, o, lse):
    ro, rl = oracle.decode(inp.q, inp.k_cache, inp.v_cache, inp.seqlens)
    live = inp.seqlens > 0
    assert_close("o", to_host(o)[live], ro[live], BF16_REL_L2, BF16_MAX_ABS)
    if lse is not None:
        gl = to_host(lse)
        assert_close("lse", gl[live], rl[live], BF16_REL_L2, BF16_MAX_ABS)
        assert np.all(np.isneginf(gl[~live]))
    assert np.all(to_host(o)[~live] == 0.0)


def test_decode_full_workload(dev):
    inp = W.make_decode_inputs()
    o, lse = run_decode(inp, dev)
    check(inp, o, lse)


def test_decode_edge_lengths(dev):
    lens = [1, 2, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1000, 2047, 2048, 0, 3]
    inp = W.make_decode_inputs(B=len(lens), H=3, seed=11, seqlens=lens)
    o, lse = run_decode(inp, dev)
    check(inp, o, lse)


def test_decode_ragged_capacity_and_no_lse(dev):
    inp = W.make_decode_inputs(B=5, T_cap=300, H=7, seed=12)
    o, lse = run_decode(inp, dev, want_lse=False)
    assert lse is None
    check(inp, o, None)


def test_decode_matches_last_forward_row(dev):
    """Decode of the token at position L-1 equals row L-1 of the training
    forward run on the same keys and values (both on the GPU)."""
    import torch
    import causal_self_attention_mha_amd as na
    L, H = 777, 2
    inp = W.make_train_inputs("d20", B=1, T=L, H=H, seed=13)
    q = to_device(inp.q_store, dev)
    k = to_device(inp.k_store, dev)
    v = to_device(inp.v_store, dev)
    o, lse = na.attn_fwd(q, k, v)
    od, ld = na.attn_decode(q[:, L - 1].contiguous(), k, v,
                            torch.tensor([L], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert_close("o", to_host(od[0]), to_host(o[0, L - 1]), 1e-2, 1e-2)
    assert_close("lse", to_host(ld[0]), to_host(lse[0, :, L - 1]), 1e-5, 1e-4)


def test_decode_many_sequences_raw_slot_order(dev):
    """More than 8192 sequences: the split kernel walks the raw (sequence,
    chunk) grid instead of the flattened list of non-empty chunks."""
    B = 8200
    rng = np.random.default_rng(14)
    lens = rng.integers(0, 70, size=B)  # includes empty sequences and chunk edges
    inp = W.make_decode_inputs(B=B, T_cap=70, H=1, seed=14, seqlens=lens)
    o, lse = run_decode(inp, dev)
    check(inp, o, lse)


def test_decode_reuses_workspace(dev):
    """Calls sharing one workspace (two different inputs, then the first again)
    each give the oracle's result."""
    import torch
    import causal_self_attention_mha_amd as na
    a = W.make_decode_inputs(B=9, T_cap=400, H=4, seed=15)
    b = W.make_decode_inputs(B=9, T_cap=400, H=4, seed=16)
    ws = torch.zeros(na.decode_workspace_bytes(9, 4, 400), dtype=torch.uint8, device=dev)
    for inp in (a, b, a):
        lens = torch.from_numpy(inp.seqlens.astype(np.int32)).to(dev)
        o, lse = na.attn_decode(to_device(inp.q_store, dev), to_device(inp.k_store, dev),
                                to_device(inp.v_store, dev), lens, workspace=ws)
        torch.cuda.synchronize()
        check(inp, o, lse)


@pytest.mark.parametrize("H,B", [(1, 100), (2, 70), (3, 60)])
def test_decode_few_heads_many_sequences(dev, H, B):
    """Workgroups of 16 H threads (fewer than a wavefront) with more sequences
    than threads: the prefix sum over the sequences' chunk counts runs in
    blocks of 16 or 32 lanes."""
    rng = np.random.default_rng(15 + H)
    lens = rng.integers(0, 300, size=B)
    inp = W.make_decode_inputs(B=B, T_cap=300, H=H, seed=15 + H, seqlens=lens)
    o, lse = run_decode(inp, dev)
    check(inp, o, lse)
