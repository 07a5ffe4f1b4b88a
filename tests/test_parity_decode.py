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


def test_decode_many_sequences_in_launch_batches(dev):
    """More than 4096 sequences: the library runs them as consecutive batches
    of split + combine launches that reuse one workspace."""
    B = 8200
    rng = np.random.default_rng(14)
    lens = rng.integers(0, 70, size=B)  # includes empty sequences and range edges
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
    than threads: the prefix sum over the sequences' visible key counts runs in
    blocks of 16 or 32 lanes."""
    rng = np.random.default_rng(15 + H)
    lens = rng.integers(0, 300, size=B)
    inp = W.make_decode_inputs(B=B, T_cap=300, H=H, seed=15 + H, seqlens=lens)
    o, lse = run_decode(inp, dev)
    check(inp, o, lse)


# ---------------------------------------------------------------- decode step with the append

APPEND_CASES = [  # B, H, Hk, T_cap, window, rope, gate
    (16, 4, 4, 300, None, False, False),
    (10, 8, 2, 500, 100, True, True),
    (64, 10, 10, 2048, None, True, False),
    (12, 6, 3, 256, None, False, True),
]


@pytest.mark.parametrize("B,H,Hk,T_cap,Wn,rope,gate", APPEND_CASES)
def test_decode_append(dev, B, H, Hk, T_cap, Wn, rope, gate):
    """na_attn_decode_append: the new token's key/value rows go to row
    L = clamp(seqlens[b], 0, T_cap - 1) (optionally normalised and rotated,
    and gated), then the query (optionally normalised and rotated at L)
    attends over rows 0 .. L; against the oracle on the cache with that row
    written.  Every other cache row is left as it was."""
    import torch
    import causal_self_attention_mha_amd as na
    from parity_util import assert_close_scaled
    rng = np.random.default_rng(500 + B + T_cap)
    lens = rng.integers(0, T_cap, size=B)
    lens[:3] = [0, T_cap - 1, T_cap + 50]              # empty, last row, clamped
    cache = W.make_decode_inputs(B=B, T_cap=T_cap, H=Hk, seed=501 + B,
                                 seqlens=np.minimum(np.maximum(lens, 1), T_cap))
    qin = W.make_decode_inputs(B=B, T_cap=1, H=H, seed=502 + B, seqlens=[1] * B)
    new = W.make_train_inputs("d20", B=B, T=1, H=Hk, seed=503 + B)
    kn_st, vn_st = new.k_store.reshape(B, Hk, 128), new.v_store.reshape(B, Hk, 128)
    kn, vn = new.k.reshape(B, Hk, 128).astype(np.float64), new.v.reshape(B, Hk, 128).astype(np.float64)
    L = np.minimum(np.maximum(lens, 0), T_cap - 1)
    c = s = None
    if rope:
        c, s = (a.astype(np.float32) for a in oracle.rope_tables(T_cap, 128))
    ve_st = g_st = None
    if gate:
        vein = W.make_train_inputs("d20", B=B, T=1, H=Hk, seed=504 + B)
        ve_st, ve = vein.k_store.reshape(B, Hk, 128), vein.k.reshape(B, Hk, 128).astype(np.float64)
        g, g_st = W.make_gate_logits(B, 1, Hk, seed=505 + B)
        g_st, g = g_st.reshape(B, Hk), g.reshape(B, Hk)
    q, kc, vc = (to_device(a, dev) for a in (qin.q_store, cache.k_store, cache.v_store))
    kc0, vc0 = to_host(kc), to_host(vc)
    args = dict(window=Wn)
    if rope:
        args["rope"] = (torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev))
    if gate:
        args["value_gate"] = (to_device(ve_st, dev), to_device(g_st, dev))
    o, lse = na.attn_decode_append(q, to_device(kn_st, dev), to_device(vn_st, dev), kc, vc,
                                   torch.from_numpy(lens.astype(np.int32)).to(dev), **args)
    torch.cuda.synchronize()
    # the oracle: the same rows through the oracle's prologue, written into the cache
    qf = qin.q.astype(np.float64)
    kr, vr = kn.copy(), vn.copy()
    if rope:
        c64, s64 = c.astype(np.float64), s.astype(np.float64)
        for b in range(B):
            p = int(L[b])
            qf[b] = oracle.qk_norm_rope_forward(qf[b][None, None], c64[p:p + 1], s64[p:p + 1])[0, 0]
            kr[b] = oracle.qk_norm_rope_forward(kn[b][None, None], c64[p:p + 1], s64[p:p + 1])[0, 0]
    if gate:
        vr = oracle.value_gate_forward(vn, ve, g)
    kcr, vcr = cache.k_cache.astype(np.float64).copy(), cache.v_cache.astype(np.float64).copy()
    for b in range(B):
        kcr[b, L[b]] = kr[b]
        vcr[b, L[b]] = vr[b]
    ro, rl = oracle.decode(qf, kcr, vcr, L + 1, window=Wn)
    assert_close("o", to_host(o), ro, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse), rl, BF16_REL_L2, BF16_MAX_ABS)
    gk, gv = to_host(kc), to_host(vc)
    rows = (np.arange(B), L)
    if rope:
        assert_close("k row", gk[rows], kr, BF16_REL_L2, BF16_MAX_ABS)
    else:
        assert np.array_equal(gk[rows], kn)
    if gate:
        assert_close_scaled("v row", gv[rows], vr, BF16_REL_L2)
    else:
        assert np.array_equal(gv[rows], vn)
    keep = np.ones((B, T_cap), dtype=bool)
    keep[rows] = False
    assert np.array_equal(gk[keep], kc0[keep]) and np.array_equal(gv[keep], vc0[keep])


def test_decode_append_many_sequences_in_launch_batches(dev):
    """The appending decode with more than 4096 sequences (several batches of
    split + combine launches) and short caches: every sequence, including ones
    whose cache was empty, sees exactly the rows before the new one plus it."""
    import torch
    import causal_self_attention_mha_amd as na
    B, H, T_cap = 8200, 1, 40
    rng = np.random.default_rng(16)
    lens = rng.integers(0, T_cap, size=B)
    cache = W.make_decode_inputs(B=B, T_cap=T_cap, H=H, seed=16, seqlens=np.maximum(lens, 1))
    new = W.make_decode_inputs(B=B, T_cap=1, H=H, seed=17, seqlens=[1] * B)
    kn, vn = to_device(new.k_store[:, 0], dev), to_device(new.v_store[:, 0], dev)
    q, kc, vc = (to_device(a, dev) for a in (cache.q_store, cache.k_store, cache.v_store))
    o, lse = na.attn_decode_append(q, kn, vn, kc, vc,
                                   torch.from_numpy(lens.astype(np.int32)).to(dev))
    torch.cuda.synchronize()
    kcr, vcr = cache.k_cache.astype(np.float64).copy(), cache.v_cache.astype(np.float64).copy()
    kcr[np.arange(B), lens] = new.k_cache[:, 0]
    vcr[np.arange(B), lens] = new.v_cache[:, 0]
    ro, rl = oracle.decode(cache.q.astype(np.float64), kcr, vcr, lens + 1)
    assert_close("o", to_host(o), ro, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse), rl, BF16_REL_L2, BF16_MAX_ABS)
