"""GPU parity of the causal attention forward and backward against the fp64
oracle, through the C ABI (Python binding -> libna_attn.so).

Small shapes are compared element by element over whole tensors; they span
several tiles, ragged tails and the degenerate T = 1.  The full training
shapes (d12, d20, d26) run in the same launch configuration the benchmark
times and are compared on every (b, h) head, which the oracle computes one
head at a time (the recompute-dq path at d20 on sampled heads).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import (BF16_MAX_ABS, BF16_REL_L2, F32_REL_L2, assert_close, to_device,
                         to_host)

pytestmark = pytest.mark.gpu


def _na():
    import causal_self_attention_mha_amd as na
    return na


def gpu_fwd_bwd(inp, dev, recompute_dq=False):
    import torch
    na = _na()
    q, k, v, do = (to_device(x, dev) for x in (inp.q_store, inp.k_store, inp.v_store,
                                               inp.do_store))
    o, lse = na.attn_fwd(q, k, v)
    dq, dk, dv, delta = na.attn_bwd(q, k, v, o, do, lse, recompute_dq=recompute_dq,
                                    return_delta=True)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)


def compare_all(inp, res, rel, mabs):
    o, lse = oracle.forward(inp.q, inp.k, inp.v)
    dq, dk, dv, delta = oracle.backward(inp.q, inp.k, inp.v, inp.do)
    for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv),
                      ("delta", delta)):
        assert_close(name, to_host(res[name]), ref, rel, mabs)


# ------------------------------------------------------------------ fp32

def test_f32_tiny_config(dev):
    """B=1, T=256, H=10 in fp32: relative L2 <= 1e-5 on every output."""
    inp = W.make_train_inputs("tiny_f32")
    compare_all(inp, gpu_fwd_bwd(inp, dev), F32_REL_L2, None)


@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (2, 33, 3), (1, 300, 2)])
def test_f32_ragged(dev, B, T, H):
    inp = W.make_train_inputs("tiny_f32", B=B, T=T, H=H, seed=1000 + T)
    compare_all(inp, gpu_fwd_bwd(inp, dev), F32_REL_L2, None)


# ------------------------------------------------------------------ bf16, small

SMALL = [(1, 1, 1), (1, 17, 2), (1, 64, 1), (1, 100, 2), (1, 128, 1), (2, 255, 1),
         (1, 257, 3), (1, 280, 2), (3, 300, 1), (1, 640, 2), (1, 1000, 1), (1, 2048, 1)]


@pytest.mark.parametrize("B,T,H", SMALL)
def test_bf16_shapes(dev, B, T, H):
    inp = W.make_train_inputs("d20", B=B, T=T, H=H, seed=2000 + 7 * T + H)
    compare_all(inp, gpu_fwd_bwd(inp, dev), BF16_REL_L2, BF16_MAX_ABS)


@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (1, 100, 2), (2, 257, 1), (1, 280, 2), (1, 1000, 1)])
def test_bf16_recompute_dq_path(dev, B, T, H):
    """The backward without a dS workspace (dq pass recomputes S and dP)."""
    inp = W.make_train_inputs("d20", B=B, T=T, H=H, seed=3000 + 7 * T + H)
    compare_all(inp, gpu_fwd_bwd(inp, dev, recompute_dq=True), BF16_REL_L2, BF16_MAX_ABS)


def test_dq_paths_agree(dev):
    """Stored-dS GEMM and recompute give the same dq up to rounding: the dK/dV
    pass that writes dS rounds dS to bf16 and scores against s log2(e) K
    rounded to bf16, where the recompute pass scales the scores in fp32, so
    P (and dS) differ by about 2^-9 relative per element; both paths are
    compared with the oracle at the bf16 tolerances elsewhere."""
    import torch
    inp = W.make_train_inputs("d20", B=1, T=700, H=2, seed=9)
    a = gpu_fwd_bwd(inp, dev)
    b = gpu_fwd_bwd(inp, dev, recompute_dq=True)
    for n in ("dk", "dv", "delta"):
        assert torch.equal(a[n], b[n]), n
    assert_close("dq paths", to_host(a["dq"]), to_host(b["dq"]), 5e-3, 2e-3)


def test_bf16_unit_scale_inputs(dev):
    """Sharper softmax: Q, K, V ~ N(0, 1) (scores of std 1), dO ~ N(0, 1)."""
    inp = W.make_train_inputs("tiny_f32", B=1, T=384, H=2, seed=77)
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    for name in ("q", "k", "v", "do"):
        bits = f32_to_bf16_bits(getattr(inp, name))
        setattr(inp, name + "_store", bits)
        setattr(inp, name, bf16_bits_to_f32(bits))
    compare_all(inp, gpu_fwd_bwd(inp, dev), BF16_REL_L2, None)


# ------------------------------------------------------------------ bf16, properties

def test_causal_independence_bitwise(dev):
    """Perturbing keys/values after position t leaves o, lse and dq of rows
    <= t bit-identical."""
    import torch
    na = _na()
    inp = W.make_train_inputs("d20", B=1, T=300, H=2, seed=5)
    r1 = gpu_fwd_bwd(inp, dev)
    t = 150
    k2, v2 = r1["k"].clone(), r1["v"].clone()
    k2[:, t + 1:] = torch.randn_like(k2[:, t + 1:], dtype=torch.float32).to(torch.bfloat16)
    v2[:, t + 1:] = torch.randn_like(v2[:, t + 1:], dtype=torch.float32).to(torch.bfloat16)
    o2, lse2 = na.attn_fwd(r1["q"], k2, v2)
    dq2, _, _ = na.attn_bwd(r1["q"], k2, v2, o2, r1["do"], lse2)
    torch.cuda.synchronize()
    assert torch.equal(r1["o"][:, :t + 1], o2[:, :t + 1])
    assert torch.equal(r1["lse"][:, :, :t + 1], lse2[:, :, :t + 1])
    assert torch.equal(r1["dq"][:, :t + 1], dq2[:, :t + 1])
    assert not torch.equal(r1["o"][:, t + 1:], o2[:, t + 1:])


def test_deterministic(dev):
    import torch
    inp = W.make_train_inputs("d20", B=2, T=700, H=3, seed=6)
    a = gpu_fwd_bwd(inp, dev)
    b = gpu_fwd_bwd(inp, dev)
    for n in ("o", "lse", "dq", "dk", "dv", "delta"):
        assert torch.equal(a[n], b[n]), n


# ------------------------------------------------------------------ bf16, full training shapes

def _sampled_heads(B, H):
    rng = np.random.default_rng(B * 1000 + H)
    pairs = {(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))}
    return sorted(pairs)


def _host32(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["d12", "d20", "d26"])
def test_full_config_every_head(dev, name):
    """Every (b, h) head of the full training shape, in the benchmark's launch
    configuration, against the fp64 oracle: each head within the bf16
    tolerances, and the whole flattened tensors too (accumulated head by
    head; the oracle computes one head at a time)."""
    inp = W.make_train_inputs(name)
    res = gpu_fwd_bwd(inp, dev)
    names = ("o", "lse", "dq", "dk", "dv", "delta")
    host = {n: _host32(res[n]) for n in names}
    del res
    B, H = inp.cfg.B, inp.cfg.H
    err2 = dict.fromkeys(names, 0.0)
    ref2 = dict.fromkeys(names, 0.0)
    worst = dict.fromkeys(names, 0.0)
    heads = [(b, h) for b in range(B) for h in range(H)]
    for c in range(0, len(heads), 16):
        chunk = heads[c:c + 16]
        fw = oracle.forward(inp.q, inp.k, inp.v, heads=chunk)
        bw = oracle.backward(inp.q, inp.k, inp.v, inp.do, heads=chunk)
        for (b, h) in chunk:
            O, L = fw[(b, h)]
            gQ, gK, gV, dl = bw[(b, h)]
            pairs = (("o", host["o"][b, :, h], O), ("lse", host["lse"][b, h], L),
                     ("dq", host["dq"][b, :, h], gQ), ("dk", host["dk"][b, :, h], gK),
                     ("dv", host["dv"][b, :, h], gV), ("delta", host["delta"][b, h], dl))
            for n, x, ref in pairs:
                x = np.asarray(x, np.float64)
                assert np.all(np.isfinite(x)), f"{name}[b={b},h={h}].{n}: non-finite"
                d = x - ref
                e2, r2, a = float(np.sum(d * d)), float(np.sum(ref * ref)), float(np.max(np.abs(d)))
                r = (e2 / r2) ** 0.5 if r2 > 0 else e2 ** 0.5
                assert r <= BF16_REL_L2 and a <= BF16_MAX_ABS, (
                    f"{name}[b={b},h={h}].{n}: rel_l2={r:.3e} max_abs={a:.3e}")
                err2[n] += e2
                ref2[n] += r2
                worst[n] = max(worst[n], a)
    for n in names:
        r = (err2[n] / ref2[n]) ** 0.5
        print(f"{name}.{n} over {len(heads)} heads: rel_l2={r:.3e} max_abs={worst[n]:.3e}")
        assert r <= BF16_REL_L2 and worst[n] <= BF16_MAX_ABS, n


def test_full_config_recompute_dq_sampled_heads(dev):
    """The backward without a dS workspace at the d20 shape, on sampled heads."""
    import torch
    name = "d20"
    inp = W.make_train_inputs(name)
    res = gpu_fwd_bwd(inp, dev, recompute_dq=True)
    for n in ("o", "dq", "dk", "dv"):
        assert bool(torch.isfinite(res[n].float()).all()), n
    assert bool(torch.isfinite(res["lse"]).all())
    heads = _sampled_heads(inp.cfg.B, inp.cfg.H)
    fw = oracle.forward(inp.q, inp.k, inp.v, heads=heads)
    bw = oracle.backward(inp.q, inp.k, inp.v, inp.do, heads=heads)
    for (b, h) in heads:
        O, L = fw[(b, h)]
        gQ, gK, gV, dl = bw[(b, h)]
        tag = f"{name}[b={b},h={h}]"
        assert_close(tag + ".o", to_host(res["o"][b, :, h]), O, BF16_REL_L2, BF16_MAX_ABS)
        assert_close(tag + ".lse", to_host(res["lse"][b, h]), L, BF16_REL_L2, BF16_MAX_ABS)
        assert_close(tag + ".dq", to_host(res["dq"][b, :, h]), gQ, BF16_REL_L2, BF16_MAX_ABS)
        assert_close(tag + ".dk", to_host(res["dk"][b, :, h]), gK, BF16_REL_L2, BF16_MAX_ABS)
        assert_close(tag + ".dv", to_host(res["dv"][b, :, h]), gV, BF16_REL_L2, BF16_MAX_ABS)
        assert_close(tag + ".delta", to_host(res["delta"][b, h]), dl, BF16_REL_L2, BF16_MAX_ABS)
