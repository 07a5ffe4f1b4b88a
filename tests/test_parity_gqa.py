"""GPU parity of grouped-query attention (H_kv key/value heads shared by H / H_kv
query heads each; query head h reads key/value head h // (H / H_kv)) against
the fp64 oracle, through the C ABI: forward, backward (dk and dv summed over
each group) and decode, plain causal and with a sliding window.  Shapes span
several tiles and ragged tails; the full d20 shape with 5 key/value heads is
compared on sampled heads."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import BF16_MAX_ABS, BF16_REL_L2, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def gqa_inputs(B, T, H, Hk, seed, cfg="d20"):
    """The seeded training inputs with key/value heads cut to the first Hk."""
    inp = W.make_train_inputs(cfg, B=B, T=T, H=H, seed=seed)
    for n in ("k", "v"):
        setattr(inp, n, np.ascontiguousarray(getattr(inp, n)[:, :, :Hk]))
        setattr(inp, n + "_store", np.ascontiguousarray(getattr(inp, n + "_store")[:, :, :Hk]))
    return inp


def gpu_fwd_bwd(inp, dev, window=None):
    import torch
    import causal_self_attention_mha_amd as na
    q, k, v, do = (to_device(x, dev) for x in (inp.q_store, inp.k_store, inp.v_store,
                                               inp.do_store))
    o, lse = na.attn_fwd(q, k, v, window=window)
    dq, dk, dv, delta = na.attn_bwd(q, k, v, o, do, lse, window=window, return_delta=True)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)


CASES = [(1, 1, 2, 1, None), (1, 100, 4, 2, None), (1, 257, 6, 2, None), (2, 300, 4, 1, None),
         (1, 640, 6, 3, None), (1, 1000, 4, 2, None), (1, 333, 4, 2, 100), (1, 700, 8, 2, 64),
         (1, 128, 4, 2, 0)]


@pytest.mark.parametrize("B,T,H,Hk,Wn", CASES)
def test_gqa_bf16_shapes(dev, B, T, H, Hk, Wn):
    inp = gqa_inputs(B, T, H, Hk, seed=5000 + 7 * T + H + Hk)
    res = gpu_fwd_bwd(inp, dev, Wn)
    assert tuple(res["dk"].shape) == (B, T, Hk, 128)
    o, lse = oracle.forward(inp.q, inp.k, inp.v, window=Wn)
    dq, dk, dv, delta = oracle.backward(inp.q, inp.k, inp.v, inp.do, window=Wn)
    for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv),
                      ("delta", delta)):
        assert_close(f"H={H} Hk={Hk} W={Wn} {name}", to_host(res[name]), ref, BF16_REL_L2,
                     BF16_MAX_ABS)


def test_gqa_one_query_head_per_group_is_mha(dev):
    """Hk = H through the grouped path's arithmetic: identical to plain MHA."""
    import torch
    import causal_self_attention_mha_amd as na
    inp = gqa_inputs(1, 300, 4, 4, seed=61)
    q, k, v, do = (to_device(x, dev) for x in (inp.q_store, inp.k_store, inp.v_store,
                                               inp.do_store))
    lib = na.load_library()
    o1, l1 = na.attn_fwd(q, k, v)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    assert lib.na_attn_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(),
                               l2.data_ptr(), 1, 300, 4, 4, 128, -1,
                               torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_full_d20_sampled_heads(dev):
    """d20 (B=32, T=2048, 10 query heads) with 5 key/value heads, sampled."""
    import torch
    B, T, H, Hk = 32, 2048, 10, 5
    inp = gqa_inputs(B, T, H, Hk, seed=None)
    res = gpu_fwd_bwd(inp, dev)
    for n in ("o", "dq", "dk", "dv"):
        assert bool(torch.isfinite(res[n].float()).all()), n
    heads = [(0, 0), (31, 9), (17, 5)]
    fw = oracle.forward(inp.q, inp.k, inp.v, heads=heads)
    bw = oracle.backward(inp.q, inp.k, inp.v, inp.do, heads=heads)
    for (b, h) in heads:
        O, L = fw[(b, h)]
        gQ = bw[(b, h)][0]
        assert_close(f"gqa d20 [b={b},h={h}].o", to_host(res["o"][b, :, h]), O, BF16_REL_L2,
                     BF16_MAX_ABS)
        assert_close(f"gqa d20 [b={b},h={h}].lse", to_host(res["lse"][b, h]), L, BF16_REL_L2,
                     BF16_MAX_ABS)
        assert_close(f"gqa d20 [b={b},h={h}].dq", to_host(res["dq"][b, :, h]), gQ, BF16_REL_L2,
                     BF16_MAX_ABS)
    kv = oracle.kv_grads(inp.q, inp.k, inp.v, inp.do, [(0, 0), (31, 4), (17, 2)])
    for (b, hk), (gK, gV) in kv.items():
        assert_close(f"gqa d20 [b={b},hk={hk}].dk", to_host(res["dk"][b, :, hk]), gK,
                     BF16_REL_L2, BF16_MAX_ABS)
        assert_close(f"gqa d20 [b={b},hk={hk}].dv", to_host(res["dv"][b, :, hk]), gV,
                     BF16_REL_L2, BF16_MAX_ABS)


@pytest.mark.parametrize("H,Hk,Wn", [(8, 2, None), (10, 5, None), (6, 1, None), (8, 4, 100)])
def test_gqa_decode(dev, H, Hk, Wn):
    import torch
    import causal_self_attention_mha_amd as na
    lens = [1, 2, 63, 64, 65, 127, 128, 129, 700, 2047, 2048, 0]
    inp = W.make_decode_inputs(B=len(lens), H=H, seed=70 + H + Hk, seqlens=lens)
    for n in ("k_cache", "v_cache"):
        setattr(inp, n, np.ascontiguousarray(getattr(inp, n)[:, :, :Hk]))
    for n in ("k_store", "v_store"):
        setattr(inp, n, np.ascontiguousarray(getattr(inp, n)[:, :, :Hk]))
    q = to_device(inp.q_store, dev)
    kc, vc = to_device(inp.k_store, dev), to_device(inp.v_store, dev)
    for b, L in enumerate(inp.seqlens):
        kc[b, int(L):] = float("nan")
        vc[b, int(L):] = float("nan")
    lensd = torch.from_numpy(inp.seqlens.astype(np.int32)).to(dev)
    o, lse = na.attn_decode(q, kc, vc, lensd, window=Wn)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(inp.q, inp.k_cache, inp.v_cache, inp.seqlens, window=Wn)
    live = inp.seqlens > 0
    assert_close("o", to_host(o)[live], ro[live], BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse)[live], rl[live], BF16_REL_L2, BF16_MAX_ABS)


@pytest.mark.parametrize("H,Hk,B,T_cap", [(4, 1, 40, 300), (2, 1, 37, 300), (10, 5, 64, 2048),
                                          (12, 3, 20, 500)])
def test_gqa_decode_many_sequences(dev, H, Hk, B, T_cap):
    """Grouped decode (one 16-lane group per key/value head serving 2 or 4
    query heads; other ratios one group per query head), ragged lengths
    U[0, T_cap], rows past each length NaN; (10, 5, 64, 2048) is the d20
    decode workload with five key/value heads."""
    import torch
    import causal_self_attention_mha_amd as na
    rng = np.random.default_rng(90 + H + Hk)
    lens = rng.integers(0, T_cap + 1, size=B)
    inp = W.make_decode_inputs(B=B, T_cap=T_cap, H=H, seed=91 + H, seqlens=lens)
    for n in ("k_cache", "v_cache", "k_store", "v_store"):
        setattr(inp, n, np.ascontiguousarray(getattr(inp, n)[:, :, :Hk]))
    q = to_device(inp.q_store, dev)
    kc, vc = to_device(inp.k_store, dev), to_device(inp.v_store, dev)
    for b, L in enumerate(inp.seqlens):
        kc[b, int(L):] = float("nan")
        vc[b, int(L):] = float("nan")
    lensd = torch.from_numpy(inp.seqlens.astype(np.int32)).to(dev)
    o, lse = na.attn_decode(q, kc, vc, lensd)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(inp.q, inp.k_cache, inp.v_cache, inp.seqlens)
    live = inp.seqlens > 0
    assert_close("o", to_host(o)[live], ro[live], BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse)[live], rl[live], BF16_REL_L2, BF16_MAX_ABS)
    assert np.all(to_host(o)[~live] == 0.0) and np.all(np.isneginf(to_host(lse)[~live]))


@pytest.mark.parametrize("cfg,B,H,Hk,Wn", [("d26", 16, 13, 1, 1024), ("d12", 16, 6, 2, 300)])
def test_gqa_window_full_shapes_sampled_heads(dev, cfg, B, H, Hk, Wn):
    """The d26 shape (13 query heads) with one key/value head and a window of
    1024, and the d12 shape with 2 key/value heads and a window of 300, at
    full size in the launch configuration the benchmark uses, on sampled
    heads."""
    import torch
    T = 2048
    inp = gqa_inputs(B, T, H, Hk, seed=None, cfg=cfg)
    res = gpu_fwd_bwd(inp, dev, window=Wn)
    for n in ("o", "dq", "dk", "dv"):
        assert bool(torch.isfinite(res[n].float()).all()), n
    heads = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    fw = oracle.forward(inp.q, inp.k, inp.v, heads=heads, window=Wn)
    bw = oracle.backward(inp.q, inp.k, inp.v, inp.do, heads=heads, window=Wn)
    for (b, h) in heads:
        O, L = fw[(b, h)]
        assert_close(f"{cfg} [b={b},h={h}].o", to_host(res["o"][b, :, h]), O, BF16_REL_L2,
                     BF16_MAX_ABS)
        assert_close(f"{cfg} [b={b},h={h}].lse", to_host(res["lse"][b, h]), L, BF16_REL_L2,
                     BF16_MAX_ABS)
        assert_close(f"{cfg} [b={b},h={h}].dq", to_host(res["dq"][b, :, h]), bw[(b, h)][0],
                     BF16_REL_L2, BF16_MAX_ABS)
    # a key/value head's gradient sums H / Hk query heads (13 at d26): one sample there
    kv_heads = [(0, 0)] if Hk == 1 else [(0, 0), (B - 1, Hk - 1)]
    kv = oracle.kv_grads(inp.q, inp.k, inp.v, inp.do, kv_heads, window=Wn)
    for (b, hk), (gK, gV) in kv.items():
        assert_close(f"{cfg} [b={b},hk={hk}].dk", to_host(res["dk"][b, :, hk]), gK,
                     BF16_REL_L2, BF16_MAX_ABS)
        assert_close(f"{cfg} [b={b},hk={hk}].dv", to_host(res["dv"][b, :, hk]), gV,
                     BF16_REL_L2, BF16_MAX_ABS)
