"""GPU parity of the prefill over a KV cache (append a chunk of T_q new key and
value rows at row L of each sequence's cache, then bottom-right causal
attention of the chunk's queries over the cache) against the fp64 oracle,
through the C ABI.  The cache after the call is compared bit for bit (the
appended rows are copies, every other row is left alone); o and lse to the
bf16 tolerances.  Cases cover an empty cache, chunk edges at 64/128 rows, a
single-token chunk, a full cache, grouped key/value heads and a window."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import BF16_MAX_ABS, BF16_REL_L2, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def make_case(B, T_q, H, Hk, T_cap, lens, seed):
    tr = W.make_train_inputs("d20", B=B, T=T_q, H=H, seed=seed)
    cache = W.make_decode_inputs(B=B, T_cap=T_cap, H=Hk, seed=seed + 1,
                                 seqlens=[max(1, min(T_cap, int(x))) for x in lens])
    kn = np.ascontiguousarray(tr.k_store[:, :, :Hk])
    vn = np.ascontiguousarray(tr.v_store[:, :, :Hk])
    return dict(q=tr.q_store, kn=kn, vn=vn, kc=cache.k_store, vc=cache.v_store,
                qf=tr.q, knf=np.ascontiguousarray(tr.k[:, :, :Hk]),
                vnf=np.ascontiguousarray(tr.v[:, :, :Hk]), kcf=cache.k_cache, vcf=cache.v_cache,
                lens=np.array(lens, dtype=np.int32))


def run(case, dev, window=None, want_lse=True):
    import torch
    import causal_self_attention_mha_amd as na
    q, kn, vn, kc, vc = (to_device(case[n], dev) for n in ("q", "kn", "vn", "kc", "vc"))
    lens = torch.from_numpy(case["lens"]).to(dev)
    o, lse = na.attn_prefill(q, kn, vn, kc, vc, lens, want_lse=want_lse, window=window)
    torch.cuda.synchronize()
    return o, lse, kc, vc


CASES = [(1, 1, 2, 2, 64, [0], None), (2, 17, 2, 2, 300, [0, 100], None),
         (2, 128, 4, 2, 600, [1, 300], None), (3, 300, 2, 1, 1024, [0, 63, 700], None),
         (1, 256, 2, 2, 2048, [1792], None), (2, 100, 2, 2, 400, [50, 299], 64),
         (2, 65, 6, 3, 500, [64, 129], 200), (1, 1, 4, 2, 2048, [2047], None)]


@pytest.mark.parametrize("B,T_q,H,Hk,T_cap,lens,Wn", CASES)
def test_prefill_shapes(dev, B, T_q, H, Hk, T_cap, lens, Wn):
    case = make_case(B, T_q, H, Hk, T_cap, lens, seed=6000 + T_q + T_cap)
    o, lse, kc, vc = run(case, dev, window=Wn)
    ro, rl, rkc, rvc = oracle.prefill(case["qf"], case["knf"], case["vnf"], case["kcf"],
                                      case["vcf"], case["lens"], window=Wn)
    assert np.array_equal(to_host(kc), rkc) and np.array_equal(to_host(vc), rvc)
    assert_close("o", to_host(o), ro, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse), rl, BF16_REL_L2, BF16_MAX_ABS)


def test_prefill_without_lse(dev):
    case = make_case(2, 50, 2, 2, 200, [10, 150], seed=61)
    o, lse, _, _ = run(case, dev, want_lse=False)
    assert lse is None
    ro, _, _, _ = oracle.prefill(case["qf"], case["knf"], case["vnf"], case["kcf"], case["vcf"],
                                 case["lens"])
    assert_close("o", to_host(o), ro, BF16_REL_L2, BF16_MAX_ABS)


def test_prefill_then_decode_agree(dev):
    """The last row of a prefilled chunk equals a decode of that token over the
    cache the prefill left behind (both on the GPU)."""
    import torch
    import causal_self_attention_mha_amd as na
    case = make_case(2, 40, 2, 2, 256, [30, 100], seed=62)
    o, lse, kc, vc = run(case, dev)
    q = to_device(case["q"], dev)
    lens = torch.from_numpy(case["lens"] + 40).to(dev)
    od, ld = na.attn_decode(q[:, -1].contiguous(), kc, vc, lens)
    torch.cuda.synchronize()
    assert_close("o", to_host(od), to_host(o[:, -1]), 1e-2, 1e-2)
    assert_close("lse", to_host(ld), to_host(lse[:, :, -1]), 1e-5, 1e-4)


def test_prefill_chat_workload_sampled_heads(dev):
    """16 sequences, a 512-token chunk each over caches of U[0, 1536] rows
    (T_cap 2048), d20 heads; sampled heads against the oracle."""
    import torch
    rng = np.random.default_rng(63)
    lens = rng.integers(0, 1537, size=16)
    case = make_case(16, 512, 10, 10, 2048, lens, seed=63)
    o, lse, kc, vc = run(case, dev)
    assert bool(torch.isfinite(o.float()).all())
    pairs = [(0, 0), (15, 9), (7, 3)]
    got = oracle.prefill(case["qf"], case["knf"], case["vnf"], case["kcf"], case["vcf"],
                         case["lens"], pairs=pairs)
    for (b, h), (O, L) in got.items():
        assert_close(f"[b={b},h={h}].o", to_host(o[b, :, h]), O, BF16_REL_L2, BF16_MAX_ABS)
        assert_close(f"[b={b},h={h}].lse", to_host(lse[b, h]), L, BF16_REL_L2, BF16_MAX_ABS)


# ---------------------------------------------------------------- prefill with the prologue folded in

ROPE_CASES = [(2, 17, 2, 2, 300, [0, 100], None), (3, 300, 2, 1, 1024, [0, 63, 700], None),
              (2, 65, 6, 3, 500, [64, 129], 200), (1, 1, 4, 2, 2048, [2047], None),
              (2, 128, 4, 2, 600, [1, 5000], None)]


@pytest.mark.parametrize("B,T_q,H,Hk,T_cap,lens,Wn", ROPE_CASES)
def test_prefill_rope_shapes(dev, B, T_q, H, Hk, T_cap, lens, Wn):
    """na_attn_prefill_rope on raw q and k_new against the oracle chain: QK norm
    + rotary embedding of q and k_new at their cache positions, then the
    prefill.  The appended key rows hold the rotated keys (bf16 tolerance),
    the value rows are copies, every other cache row is left as it was."""
    import torch
    import causal_self_attention_mha_amd as na
    case = make_case(B, T_q, H, Hk, T_cap, lens, seed=6500 + T_q + T_cap)
    c, s = oracle.rope_tables(T_cap, 128)
    c, s = c.astype(np.float32), s.astype(np.float32)
    q, kn, vn, kc, vc = (to_device(case[n], dev) for n in ("q", "kn", "vn", "kc", "vc"))
    kc0 = to_host(kc)
    lensd = torch.from_numpy(case["lens"]).to(dev)
    o, lse = na.attn_prefill(q, kn, vn, kc, vc, lensd, window=Wn,
                             rope=(torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)))
    torch.cuda.synchronize()
    starts = [min(max(int(x), 0), T_cap - T_q) for x in case["lens"]]
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    qr = np.concatenate([oracle.qk_norm_rope_forward(case["qf"][b:b + 1], c64[L:L + T_q],
                                                     s64[L:L + T_q]) for b, L in enumerate(starts)])
    kr = np.concatenate([oracle.qk_norm_rope_forward(case["knf"][b:b + 1], c64[L:L + T_q],
                                                     s64[L:L + T_q]) for b, L in enumerate(starts)])
    # the device clamps cache_lens to [0, T_cap - T_q]; the oracle takes the clamped rows
    ro, rl, rkc, rvc = oracle.prefill(qr, kr, case["vnf"], case["kcf"], case["vcf"],
                                      np.array(starts), window=Wn)
    assert_close("o", to_host(o), ro, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse), rl, BF16_REL_L2, BF16_MAX_ABS)
    gk, gv = to_host(kc), to_host(vc)
    assert np.array_equal(gv, rvc)
    for b, L in enumerate(starts):
        assert_close(f"k_cache[{b}] appended", gk[b, L:L + T_q], rkc[b, L:L + T_q], BF16_REL_L2,
                     BF16_MAX_ABS)
        assert np.array_equal(gk[b, :L], kc0[b, :L]) and np.array_equal(gk[b, L + T_q:],
                                                                        kc0[b, L + T_q:])


def test_prefill_rope_matches_prologue_then_prefill(dev):
    """The folded call against the two-step path on the GPU (na_qk_norm_rope_fwd
    with pos_offset = cache_lens, then na_attn_prefill): the same results up to
    the rounding order of the normalisation's sum (a consistency check; parity
    with the oracle is the test above)."""
    import torch
    import causal_self_attention_mha_amd as na
    case = make_case(3, 200, 4, 2, 800, [0, 350, 9999], seed=64)
    c, s = (torch.from_numpy(a.astype(np.float32)).to(dev) for a in oracle.rope_tables(800, 128))
    lensd = torch.from_numpy(case["lens"]).to(dev)
    q, kn, vn = (to_device(case[n], dev) for n in ("q", "kn", "vn"))
    kc1, vc1 = to_device(case["kc"], dev), to_device(case["vc"], dev)
    kc2, vc2 = kc1.clone(), vc1.clone()
    o1, l1 = na.attn_prefill(q, kn, vn, kc1, vc1, lensd, rope=(c, s))
    qr, kr = na.qk_norm_rope_fwd(q, kn, c, s, pos_offset=lensd)
    o2, l2 = na.attn_prefill(qr, kr, vn, kc2, vc2, lensd)
    torch.cuda.synchronize()
    # the two paths may round an element of the rotated q or k to different
    # bf16 neighbours, so they are compared to the bf16 bound
    assert_close("o", to_host(o1), to_host(o2), BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(l1), to_host(l2), BF16_REL_L2, BF16_MAX_ABS)
    assert_close("k_cache", to_host(kc1), to_host(kc2), BF16_REL_L2, BF16_MAX_ABS)
    assert torch.equal(vc1, vc2)


@pytest.mark.parametrize("B,T_q,H,Hk,T_cap,lens", [(2, 70, 4, 2, 400, [0, 250]),
                                                   (3, 129, 2, 2, 700, [5, 300, 571])])
def test_prefill_rope_value_gate(dev, B, T_q, H, Hk, T_cap, lens):
    """na_attn_prefill_rope with the value-embedding gate: the appended value
    rows are v_new + 3 sigmoid(g) ve (they reach past 8, so the scaled bf16
    bound), and attention uses them."""
    import torch
    import causal_self_attention_mha_amd as na
    from parity_util import assert_close_scaled
    case = make_case(B, T_q, H, Hk, T_cap, lens, seed=6600 + T_q)
    ve_in = W.make_train_inputs("d20", B=B, T=T_q, H=Hk, seed=6601 + T_q)
    g, g_st = W.make_gate_logits(B, T_q, Hk, seed=6602 + T_q)
    c, s = (a.astype(np.float32) for a in oracle.rope_tables(T_cap, 128))
    q, kn, vn, kc, vc = (to_device(case[n], dev) for n in ("q", "kn", "vn", "kc", "vc"))
    ve, gt = to_device(ve_in.k_store, dev), to_device(g_st, dev)
    lensd = torch.from_numpy(case["lens"]).to(dev)
    o, lse = na.attn_prefill(q, kn, vn, kc, vc, lensd, rope=(torch.from_numpy(c).to(dev),
                                                               torch.from_numpy(s).to(dev)),
                             value_gate=(ve, gt))
    torch.cuda.synchronize()
    starts = [min(max(int(x), 0), T_cap - T_q) for x in case["lens"]]
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    qr = np.concatenate([oracle.qk_norm_rope_forward(case["qf"][b:b + 1], c64[L:L + T_q],
                                                     s64[L:L + T_q]) for b, L in enumerate(starts)])
    kr = np.concatenate([oracle.qk_norm_rope_forward(case["knf"][b:b + 1], c64[L:L + T_q],
                                                     s64[L:L + T_q]) for b, L in enumerate(starts)])
    vg = oracle.value_gate_forward(case["vnf"], ve_in.k.astype(np.float64), g)
    ro, rl, rkc, rvc = oracle.prefill(qr, kr, vg, case["kcf"], case["vcf"], np.array(starts))
    assert_close("o", to_host(o), ro, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse), rl, BF16_REL_L2, BF16_MAX_ABS)
    gv = to_host(vc)
    for b, L in enumerate(starts):
        assert_close_scaled(f"v_cache[{b}] appended", gv[b, L:L + T_q], rvc[b, L:L + T_q],
                            BF16_REL_L2)
        assert np.array_equal(gv[b, :L], case["vcf"][b, :L])
