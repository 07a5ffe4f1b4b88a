"""GPU parity of the sliding-window (banded causal) entry points against the
fp64 oracle with the same window, through the C ABI: key j is visible to
query i iff i - W <= j <= i; decode sees keys L - 1 - W .. L - 1.

Windows are chosen around the kernels' tile edges (32-row blocks, 64-row
tiles, 128-key workgroup tiles) and the degenerate W = 0; lengths are ragged.
Cache rows outside each sequence's window are filled with NaN, so a read of
them shows up.  The full d20 shape runs at W = 1024 on sampled heads."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import BF16_MAX_ABS, BF16_REL_L2, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def _na():
    import causal_self_attention_mha_amd as na
    return na


def gpu_fwd_bwd(inp, dev, window, recompute_dq=False):
    import torch
    na = _na()
    q, k, v, do = (to_device(x, dev) for x in (inp.q_store, inp.k_store, inp.v_store,
                                               inp.do_store))
    o, lse = na.attn_fwd(q, k, v, window=window)
    dq, dk, dv, delta = na.attn_bwd(q, k, v, o, do, lse, window=window, recompute_dq=recompute_dq,
                                    return_delta=True)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)


CASES = [(1, 1, 1, 0), (1, 100, 2, 0), (1, 100, 2, 1), (1, 333, 2, 31), (2, 257, 1, 32),
         (1, 300, 2, 63), (1, 300, 1, 64), (1, 700, 2, 100), (1, 640, 1, 127), (2, 500, 1, 128),
         (1, 1000, 1, 200), (1, 2048, 1, 1024), (1, 333, 2, 331)]


@pytest.mark.parametrize("B,T,H,Wn", CASES)
def test_window_bf16_shapes(dev, B, T, H, Wn):
    inp = W.make_train_inputs("d20", B=B, T=T, H=H, seed=4000 + 7 * T + H + Wn)
    res = gpu_fwd_bwd(inp, dev, Wn)
    o, lse = oracle.forward(inp.q, inp.k, inp.v, window=Wn)
    dq, dk, dv, delta = oracle.backward(inp.q, inp.k, inp.v, inp.do, window=Wn)
    for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv),
                      ("delta", delta)):
        assert_close(f"W={Wn} {name}", to_host(res[name]), ref, BF16_REL_L2, BF16_MAX_ABS)


@pytest.mark.parametrize("B,T,H,Wn", [(1, 100, 2, 0), (1, 333, 2, 31), (2, 257, 1, 32),
                                      (1, 300, 1, 64), (1, 700, 2, 100), (2, 500, 1, 128),
                                      (1, 2048, 1, 1024), (1, 333, 2, 331)])
def test_window_recompute_dq(dev, B, T, H, Wn):
    """The windowed backward without a dS workspace: the dq pass recomputes S
    and dP over the band (both selects in every block); dk, dv, delta are the
    same pass as with the workspace."""
    import torch
    inp = W.make_train_inputs("d20", B=B, T=T, H=H, seed=4500 + 7 * T + H + Wn)
    res = gpu_fwd_bwd(inp, dev, Wn, recompute_dq=True)
    dq, dk, dv, delta = oracle.backward(inp.q, inp.k, inp.v, inp.do, window=Wn)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv), ("delta", delta)):
        assert_close(f"W={Wn} {name}", to_host(res[name]), ref, BF16_REL_L2, BF16_MAX_ABS)
    ws = gpu_fwd_bwd(inp, dev, Wn)
    for n in ("dk", "dv", "delta"):
        assert torch.equal(res[n], ws[n]), n


def test_window_recompute_dq_grouped(dev):
    """The same with grouped key/value heads (4 query heads, 2 key/value heads)."""
    import torch
    na = _na()
    inp = W.make_train_inputs("d20", B=1, T=400, H=4, seed=4601)
    q, k, v, do = (to_device(x, dev) for x in (inp.q_store, inp.k_store, inp.v_store,
                                               inp.do_store))
    k2, v2 = k[:, :, :2].contiguous(), v[:, :, :2].contiguous()
    o, lse = na.attn_fwd(q, k2, v2, window=90)
    dq, dk, dv = na.attn_bwd(q, k2, v2, o, do, lse, window=90, recompute_dq=True)
    dq_ws, dk_ws, dv_ws = na.attn_bwd(q, k2, v2, o, do, lse, window=90)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk_ws) and torch.equal(dv, dv_ws)
    kk = inp.k[:, :, :2]
    vv = inp.v[:, :, :2]
    rdq, _, _, _ = oracle.backward(inp.q, np.repeat(kk, 2, axis=2), np.repeat(vv, 2, axis=2),
                                   inp.do, window=90)
    assert_close("dq", to_host(dq), rdq, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dq paths", to_host(dq), to_host(dq_ws), 5e-3, 2e-3)


def test_window_covering_every_key_is_the_plain_call(dev):
    """W >= T - 1 reaches key 0 from every row: bitwise the plain causal call."""
    import torch
    na = _na()
    inp = W.make_train_inputs("d20", B=1, T=300, H=2, seed=41)
    a = gpu_fwd_bwd(inp, dev, 299)
    q, k, v, do = a["q"], a["k"], a["v"], a["do"]
    o, lse = na.attn_fwd(q, k, v)
    dq, dk, dv, delta = na.attn_bwd(q, k, v, o, do, lse, return_delta=True)
    torch.cuda.synchronize()
    for n, x in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(a[n], x), n


def test_window_zero_copies_v(dev):
    """W = 0: each query sees only itself, so o = v exactly (P = 1)."""
    import torch
    inp = W.make_train_inputs("d20", B=1, T=200, H=2, seed=42)
    res = gpu_fwd_bwd(inp, dev, 0)
    assert torch.equal(res["o"], res["v"])


def test_window_ignores_keys_before_the_band(dev):
    """Keys more than W rows before a query do not affect its output."""
    import torch
    na = _na()
    inp = W.make_train_inputs("d20", B=1, T=400, H=1, seed=43)
    Wn, t = 90, 250
    r1 = gpu_fwd_bwd(inp, dev, Wn)
    k2, v2 = r1["k"].clone(), r1["v"].clone()
    k2[:, :t - Wn] = torch.randn_like(k2[:, :t - Wn], dtype=torch.float32).to(torch.bfloat16)
    v2[:, :t - Wn] = torch.randn_like(v2[:, :t - Wn], dtype=torch.float32).to(torch.bfloat16)
    o2, lse2 = na.attn_fwd(r1["q"], k2, v2, window=Wn)
    torch.cuda.synchronize()
    assert torch.equal(r1["o"][:, t:], o2[:, t:])
    assert torch.equal(r1["lse"][:, :, t:], lse2[:, :, t:])


def test_window_full_d20_sampled_heads(dev):
    """d20 (B=32, T=2048, H=10) at W = 1024, in the benchmark's launch
    configuration, on sampled heads."""
    import torch
    inp = W.make_train_inputs("d20")
    Wn = 1024
    res = gpu_fwd_bwd(inp, dev, Wn)
    for n in ("o", "dq", "dk", "dv"):
        assert bool(torch.isfinite(res[n].float()).all()), n
    heads = [(0, 0), (31, 9), (17, 4)]
    fw = oracle.forward(inp.q, inp.k, inp.v, heads=heads, window=Wn)
    bw = oracle.backward(inp.q, inp.k, inp.v, inp.do, heads=heads, window=Wn)
    for (b, h) in heads:
        O, L = fw[(b, h)]
        gQ, gK, gV, _ = bw[(b, h)]
        for n, ref, x in (("o", O, res["o"][b, :, h]), ("lse", L, res["lse"][b, h]),
                          ("dq", gQ, res["dq"][b, :, h]), ("dk", gK, res["dk"][b, :, h]),
                          ("dv", gV, res["dv"][b, :, h])):
            assert_close(f"d20 W={Wn} [b={b},h={h}].{n}", to_host(x), ref, BF16_REL_L2,
                         BF16_MAX_ABS)


# ------------------------------------------------------------------ decode

def run_decode(inp, dev, window):
    import torch
    na = _na()
    q = to_device(inp.q_store, dev)
    kc = to_device(inp.k_store, dev)
    vc = to_device(inp.v_store, dev)
    for b, L in enumerate(inp.seqlens):
        L = int(L)
        kc[b, L:] = float("nan")
        vc[b, L:] = float("nan")
        j0 = max(0, L - 1 - window)
        kc[b, :j0] = float("nan")
        vc[b, :j0] = float("nan")
    lens = torch.from_numpy(inp.seqlens.astype(np.int32)).to(dev)
    o, lse = na.attn_decode(q, kc, vc, lens, window=window)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("Wn", [0, 1, 5, 63, 64, 65, 127, 300, 2046])
def test_window_decode_edge_lengths(dev, Wn):
    lens = [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 700, 1000, 2047, 2048, 0]
    inp = W.make_decode_inputs(B=len(lens), H=3, seed=50 + Wn, seqlens=lens)
    o, lse = run_decode(inp, dev, Wn)
    ro, rl = oracle.decode(inp.q, inp.k_cache, inp.v_cache, inp.seqlens, window=Wn)
    live = inp.seqlens > 0
    assert_close(f"W={Wn} o", to_host(o)[live], ro[live], BF16_REL_L2, BF16_MAX_ABS)
    gl = to_host(lse)
    assert_close(f"W={Wn} lse", gl[live], rl[live], BF16_REL_L2, BF16_MAX_ABS)
    assert np.all(np.isneginf(gl[~live])) and np.all(to_host(o)[~live] == 0.0)


def test_window_decode_full_workload(dev):
    """The d20 decode workload (64 sequences, lengths U[1, 2048]) at W = 1024."""
    inp = W.make_decode_inputs()
    o, lse = run_decode(inp, dev, 1024)
    ro, rl = oracle.decode(inp.q, inp.k_cache, inp.v_cache, inp.seqlens, window=1024)
    assert_close("o", to_host(o), ro, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse), rl, BF16_REL_L2, BF16_MAX_ABS)


def test_window_decode_many_sequences_raw_slot_order(dev):
    """More than 4096 sequences (several split/combine launch pairs) with a window."""
    B = 8200
    rng = np.random.default_rng(51)
    lens = rng.integers(0, 200, size=B)
    inp = W.make_decode_inputs(B=B, T_cap=200, H=1, seed=51, seqlens=lens)
    o, lse = run_decode(inp, dev, 70)
    ro, rl = oracle.decode(inp.q, inp.k_cache, inp.v_cache, inp.seqlens, window=70)
    live = inp.seqlens > 0
    assert_close("o", to_host(o)[live], ro[live], BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse)[live], rl[live], BF16_REL_L2, BF16_MAX_ABS)
