"""GPU parity of the attention prologue (RMS normalisation + rotary embedding
of the query and key heads, and the value-embedding gate, forward and
backward) against the fp64 oracle, through the C ABI.  Cases: a single row, ragged T, grouped key heads, per
sequence position offsets (clamped into the table), tables of standard
RoPE angles and of random angles, all-zero rows, large magnitudes, the d20
training shape on sampled positions, and the prologue chained with the
attention forward and backward."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import (BF16_MAX_ABS, BF16_REL_L2, assert_close, assert_close_scaled, to_device,
                         to_host)

pytestmark = pytest.mark.gpu

EPS = 1e-6


def tables(kind, T_tab, seed):
    if kind == "rope":
        c, s = oracle.rope_tables(T_tab, 128)
        return c.astype(np.float32), s.astype(np.float32)
    return W.make_angle_tables(T_tab, 64, seed)


def positions(B, T, T_tab, offs):
    if offs is None:
        return [0] * B
    return [min(max(int(o), 0), T_tab - T) for o in offs]


def oracle_pair(xq, xk, gq, gk, c, s, starts, eps=EPS):
    """Oracle forward and backward of q and k, sequence b at positions
    starts[b] .. starts[b] + T - 1 of the tables."""
    T = xq.shape[1]
    out = {n: [] for n in ("yq", "yk", "dq", "dk")}
    for b, p0 in enumerate(starts):
        cb, sb = c[p0:p0 + T].astype(np.float64), s[p0:p0 + T].astype(np.float64)
        out["yq"].append(oracle.qk_norm_rope_forward(xq[b:b + 1], cb, sb, eps))
        out["yk"].append(oracle.qk_norm_rope_forward(xk[b:b + 1], cb, sb, eps))
        out["dq"].append(oracle.qk_norm_rope_backward(xq[b:b + 1], gq[b:b + 1], cb, sb, eps))
        out["dk"].append(oracle.qk_norm_rope_backward(xk[b:b + 1], gk[b:b + 1], cb, sb, eps))
    return {n: np.concatenate(v, axis=0) for n, v in out.items()}


def make_case(B, T, H, Hk, seed, scale=1.0, zero_rows=0):
    tr = W.make_train_inputs("d20", B=B, T=T, H=H, seed=seed)
    st = {"q": tr.q_store, "k": np.ascontiguousarray(tr.k_store[:, :, :Hk]),
          "gq": tr.do_store, "gk": np.ascontiguousarray(tr.v_store[:, :, :Hk])}
    val = {"q": tr.q.astype(np.float64), "k": tr.k[:, :, :Hk].astype(np.float64),
           "gq": tr.do.astype(np.float64), "gk": tr.v[:, :, :Hk].astype(np.float64)}
    if scale != 1.0:   # a power of two keeps the bf16 values exact
        for n in ("q", "k"):
            val[n] = val[n] * scale
            st[n] = W.f32_to_bf16_bits(val[n].astype(np.float32))
    if zero_rows:
        rng = np.random.default_rng(seed + 7)
        for n in ("q", "k"):
            flat_v = val[n].reshape(-1, 128)
            flat_s = st[n].reshape(-1, 128)
            idx = rng.choice(flat_v.shape[0], size=zero_rows, replace=False)
            flat_v[idx] = 0.0
            flat_s[idx] = 0
    return st, val


def run_gpu(st, c, s, offs, dev, eps=EPS, host=True):
    import torch
    import causal_self_attention_mha_amd as na
    q, k, gq, gk = (to_device(st[n], dev) for n in ("q", "k", "gq", "gk"))
    ct, sn = torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)
    po = None if offs is None else torch.tensor(offs, dtype=torch.int32, device=dev)
    yq, yk = na.qk_norm_rope_fwd(q, k, ct, sn, pos_offset=po, eps=eps)
    dq, dk = na.qk_norm_rope_bwd(q, k, gq, gk, ct, sn, pos_offset=po, eps=eps)
    torch.cuda.synchronize()
    out = {"yq": yq, "yk": yk, "dq": dq, "dk": dk}
    return {n: to_host(t) for n, t in out.items()} if host else out


CASES = [  # B, T, H, Hk, T_tab, offsets, table kind
    (1, 1, 1, 1, 1, None, "rope"),
    (2, 37, 3, 1, 64, None, "rope"),
    (2, 100, 10, 10, 100, None, "rope"),
    (3, 50, 4, 2, 300, [0, 17, 290], "rope"),
    (2, 64, 2, 2, 64, [-5, 10], "random"),
    (4, 129, 6, 3, 2048, [1919, 0, 1000, 5000], "random"),
]


@pytest.mark.parametrize("B,T,H,Hk,T_tab,offs,kind", CASES)
def test_prologue_shapes(dev, B, T, H, Hk, T_tab, offs, kind):
    st, val = make_case(B, T, H, Hk, seed=7000 + T + H)
    c, s = tables(kind, T_tab, seed=T_tab)
    got = run_gpu(st, c, s, offs, dev)
    ref = oracle_pair(val["q"], val["k"], val["gq"], val["gk"], c, s, positions(B, T, T_tab, offs))
    for n in ("yq", "yk", "dq", "dk"):
        assert_close(n, got[n], ref[n], BF16_REL_L2, BF16_MAX_ABS)


def test_prologue_zero_rows_and_large_values(dev):
    """All-zero head rows: zero outputs, and the gradient R^T dy / sqrt(eps)
    (the normalisation's slope at zero, values near 1000 |dy|, so compared by
    relative L2 only); rows scaled by 64 normalise like unscaled ones."""
    c, s = tables("rope", 80, 0)
    st, val = make_case(2, 80, 4, 2, seed=71, zero_rows=40)
    got = run_gpu(st, c, s, None, dev)
    ref = oracle_pair(val["q"], val["k"], val["gq"], val["gk"], c, s, [0, 0])
    for y, d, x in (("yq", "dq", "q"), ("yk", "dk", "k")):
        z = np.all(val[x] == 0, axis=-1)
        assert z.sum() > 0 and np.all(got[y][z] == 0)
        assert_close(f"{d} zero rows", got[d][z], ref[d][z], BF16_REL_L2)
        assert_close(y, got[y], ref[y], BF16_REL_L2, BF16_MAX_ABS)
        assert_close(f"{d} other rows", got[d][~z], ref[d][~z], BF16_REL_L2, BF16_MAX_ABS)
    st2, val2 = make_case(2, 80, 4, 2, seed=72, scale=64.0)
    got2 = run_gpu(st2, c, s, None, dev)
    ref2 = oracle_pair(val2["q"], val2["k"], val2["gq"], val2["gk"], c, s, [0, 0])
    for n in ("yq", "yk", "dq", "dk"):
        assert_close(n, got2[n], ref2[n], BF16_REL_L2, BF16_MAX_ABS)


def test_prologue_d20_sampled(dev):
    """The d20 training shape (B=32, T=2048, H=10, D=128) with standard RoPE
    tables, in the launch the benchmark times; the oracle checks 96 sampled
    (b, t) positions, every head of each."""
    B, T, H = 32, 2048, 10
    tr = W.make_train_inputs("d20", seed=20)
    assert tr.q.shape == (B, T, H, 128)
    c, s = tables("rope", T, 0)
    st = {"q": tr.q_store, "k": tr.k_store, "gq": tr.do_store, "gk": tr.v_store}
    got = run_gpu(st, c, s, None, dev, host=False)
    rng = np.random.default_rng(5)
    bs, ts = rng.integers(0, B, 96), rng.integers(0, T, 96)
    ts[:4] = [0, 1, T - 1, T // 2]
    for b, t in zip(bs, ts):
        sl = (slice(b, b + 1), slice(t, t + 1))
        ref = oracle_pair(tr.q[sl].astype(np.float64), tr.k[sl].astype(np.float64),
                          tr.do[sl].astype(np.float64), tr.v[sl].astype(np.float64),
                          c[t:t + 1], s[t:t + 1], [0])
        for n in ("yq", "yk", "dq", "dk"):
            assert_close(f"{n}[{b},{t}]", to_host(got[n][sl]), ref[n], BF16_REL_L2,
                         BF16_MAX_ABS)


def test_prologue_chained_with_attention(dev):
    """prologue -> attention forward -> attention backward -> prologue backward
    on the GPU against the same chain through the oracle: o and the gradients
    of the pre-normalisation q and k."""
    import torch
    import causal_self_attention_mha_amd as na
    B, T, H = 2, 96, 2
    tr = W.make_train_inputs("d20", B=B, T=T, H=H, seed=77)
    c, s = tables("rope", T, 0)
    q, k, v, do = (to_device(a, dev) for a in (tr.q_store, tr.k_store, tr.v_store, tr.do_store))
    ct, sn = torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)
    qr, kr = na.qk_norm_rope_fwd(q, k, ct, sn)
    o, lse = na.attn_fwd(qr, kr, v)
    dqr, dkr, dv = na.attn_bwd(qr, kr, v, o, do, lse)
    dq, dk = na.qk_norm_rope_bwd(q, k, dqr, dkr, ct, sn)
    torch.cuda.synchronize()
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    rq = oracle.qk_norm_rope_forward(tr.q.astype(np.float64), c64, s64, EPS)
    rk = oracle.qk_norm_rope_forward(tr.k.astype(np.float64), c64, s64, EPS)
    ro, rl = oracle.forward(rq, rk, tr.v)
    rdq, rdk, rdv, _ = oracle.backward(rq, rk, tr.v, tr.do)
    assert_close("o", to_host(o), ro, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dv", to_host(dv), rdv, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dq", to_host(dq),
                 oracle.qk_norm_rope_backward(tr.q.astype(np.float64), rdq, c64, s64, EPS),
                 BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dk", to_host(dk),
                 oracle.qk_norm_rope_backward(tr.k.astype(np.float64), rdk, c64, s64, EPS),
                 BF16_REL_L2, BF16_MAX_ABS)


def run_value_gate(v_st, ve_st, g_st, dy_st, dev):
    import torch
    import causal_self_attention_mha_amd as na
    v, ve, dy = (to_device(a, dev) for a in (v_st, ve_st, dy_st))
    g = to_device(g_st, dev)
    out = na.value_gate_fwd(v, ve, g)
    dve, dg = na.value_gate_bwd(ve, g, dy)
    torch.cuda.synchronize()
    return to_host(out), to_host(dve), to_host(dg)


@pytest.mark.parametrize("B,T,Hk", [(1, 1, 1), (2, 37, 3), (3, 100, 5), (2, 65, 10)])
def test_value_gate_shapes(dev, B, T, Hk):
    """v_out reaches |v| + 3 |ve| (past 8 at these scales), so its element bound
    grows with the magnitude (one bf16 step); dve and dgate stay small."""
    tr = W.make_train_inputs("d20", B=B, T=T, H=Hk, seed=8000 + T)
    g, g_st = W.make_gate_logits(B, T, Hk, seed=T)
    out, dve, dg = run_value_gate(tr.v_store, tr.k_store, g_st, tr.do_store, dev)
    v, ve, dy = (a.astype(np.float64) for a in (tr.v, tr.k, tr.do))
    assert_close_scaled("v_out", out, oracle.value_gate_forward(v, ve, g), BF16_REL_L2)
    rdve, rdg = oracle.value_gate_backward(ve, g, dy)
    assert_close("dve", dve, rdve, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dgate", dg, rdg, BF16_REL_L2, BF16_MAX_ABS)


def test_value_gate_saturated_logits_and_d20(dev):
    """Logits of +-60 saturate the gate at 0 and 3 (finite, gate gradient 0);
    then the d20 key/value shape (B=32, T=2048, H_kv=10), compared whole."""
    B, T, Hk = 2, 40, 2
    tr = W.make_train_inputs("d20", B=B, T=T, H=Hk, seed=81)
    g = np.where(np.arange(B * T * Hk).reshape(B, T, Hk) % 2 == 0, 60.0, -60.0).astype(np.float32)
    g_st = W.f32_to_bf16_bits(g)
    out, dve, dg = run_value_gate(tr.v_store, tr.k_store, g_st, tr.do_store, dev)
    v, ve, dy = (a.astype(np.float64) for a in (tr.v, tr.k, tr.do))
    assert_close_scaled("v_out", out, oracle.value_gate_forward(v, ve, g), BF16_REL_L2)
    assert np.all(np.abs(dg) < 1e-20)
    tr = W.make_train_inputs("d20", seed=82)
    B, T, Hk = tr.q.shape[:3]
    g, g_st = W.make_gate_logits(B, T, Hk, seed=83)
    out, dve, dg = run_value_gate(tr.v_store, tr.k_store, g_st, tr.do_store, dev)
    v, ve, dy = (a.astype(np.float64) for a in (tr.v, tr.k, tr.do))
    assert_close_scaled("v_out d20", out, oracle.value_gate_forward(v, ve, g), BF16_REL_L2)
    rdve, rdg = oracle.value_gate_backward(ve, g, dy)
    assert_close("dve d20", dve, rdve, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dgate d20", dg, rdg, BF16_REL_L2, BF16_MAX_ABS)


@pytest.mark.parametrize("B,T,H,Hk,Wn", [(2, 96, 2, 2, None), (2, 300, 4, 2, None),
                                         (1, 257, 2, 2, 64), (3, 130, 6, 3, 40)])
def test_bwd_with_prologue_folded_in(dev, B, T, H, Hk, Wn):
    """na_attn_bwd_rope (the prologue's backward in the dQ and dK/dV epilogues)
    against the oracle chain: prologue -> attention forward -> attention
    backward -> prologue backward; dv unchanged by the prologue."""
    import torch
    import causal_self_attention_mha_amd as na
    tr = W.make_train_inputs("d20", B=B, T=T, H=H, seed=770 + T)
    kv = lambda a: np.ascontiguousarray(a[:, :, :Hk])  # noqa: E731
    c, s = tables("rope", T, 0)
    q_raw, k_raw = to_device(tr.q_store, dev), to_device(kv(tr.k_store), dev)
    v, do = to_device(kv(tr.v_store), dev), to_device(tr.do_store, dev)
    ct, sn = torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)
    qr, kr = na.qk_norm_rope_fwd(q_raw, k_raw, ct, sn)
    o, lse = na.attn_fwd(qr, kr, v, window=Wn)
    dq, dk, dv = na.attn_bwd(qr, kr, v, o, do, lse, window=Wn, rope=(q_raw, k_raw, ct, sn))
    torch.cuda.synchronize()
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    xq, xk = tr.q.astype(np.float64), kv(tr.k).astype(np.float64)
    rq = oracle.qk_norm_rope_forward(xq, c64, s64, EPS)
    rk = oracle.qk_norm_rope_forward(xk, c64, s64, EPS)
    rdq, rdk, rdv, _ = oracle.backward(rq, rk, kv(tr.v), tr.do, window=Wn)
    assert_close("dv", to_host(dv), rdv, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dq", to_host(dq), oracle.qk_norm_rope_backward(xq, rdq, c64, s64, EPS),
                 BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dk", to_host(dk), oracle.qk_norm_rope_backward(xk, rdk, c64, s64, EPS),
                 BF16_REL_L2, BF16_MAX_ABS)


@pytest.mark.parametrize("B,T,H,Hk,Wn", [(2, 96, 2, 2, None), (2, 300, 4, 2, None),
                                         (1, 257, 2, 2, 64)])
def test_bwd_with_prologue_and_gate_folded_in(dev, B, T, H, Hk, Wn):
    """na_attn_bwd_rope with the value-embedding gate folded in as well: the
    attention ran on v' = v + 3 sigmoid(g) ve.  dq, dk, dv against the oracle
    chain (prologue, gate -> attention -> backward -> prologue backward), dve
    and dgate against the oracle's gate backward of the oracle dv, and bit for
    bit against the separate gate backward kernel run on the folded dv (the
    same bf16 dv, the same arithmetic)."""
    import torch
    import causal_self_attention_mha_amd as na
    tr = W.make_train_inputs("d20", B=B, T=T, H=H, seed=990 + T)
    kv = lambda a: np.ascontiguousarray(a[:, :, :Hk])  # noqa: E731
    g, g_st = W.make_gate_logits(B, T, Hk, seed=91 + T)
    c, s = tables("rope", T, 0)
    q_raw, k_raw = to_device(tr.q_store, dev), to_device(kv(tr.k_store), dev)
    v_in, do = to_device(kv(tr.v_store), dev), to_device(tr.do_store, dev)
    ve, gd = to_device(kv(tr.k_store[:, ::-1]), dev), to_device(g_st, dev)
    ct, sn = torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)
    qr, kr = na.qk_norm_rope_fwd(q_raw, k_raw, ct, sn)
    v = na.value_gate_fwd(v_in, ve, gd)
    o, lse = na.attn_fwd(qr, kr, v, window=Wn)
    dq, dk, dv, dve, dg = na.attn_bwd(qr, kr, v, o, do, lse, window=Wn,
                                      rope=(q_raw, k_raw, ct, sn), value_gate=(ve, gd))
    dve2, dg2 = na.value_gate_bwd(ve, gd, dv)
    torch.cuda.synchronize()
    assert torch.equal(dve, dve2) and torch.equal(dg, dg2)
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    xq, xk = tr.q.astype(np.float64), kv(tr.k).astype(np.float64)
    ve64 = kv(tr.k[:, ::-1]).astype(np.float64)
    rq = oracle.qk_norm_rope_forward(xq, c64, s64, EPS)
    rk = oracle.qk_norm_rope_forward(xk, c64, s64, EPS)
    rv = oracle.value_gate_forward(kv(tr.v), ve64, g)
    rdq, rdk, rdv, _ = oracle.backward(rq, rk, rv, tr.do, window=Wn)
    assert_close("dv", to_host(dv), rdv, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dq", to_host(dq), oracle.qk_norm_rope_backward(xq, rdq, c64, s64, EPS),
                 BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dk", to_host(dk), oracle.qk_norm_rope_backward(xk, rdk, c64, s64, EPS),
                 BF16_REL_L2, BF16_MAX_ABS)
    rdve, rdg = oracle.value_gate_backward(ve64, g, rdv)
    assert_close("dve", to_host(dve), rdve, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dgate", to_host(dg), rdg, BF16_REL_L2, BF16_MAX_ABS)


def test_bwd_with_prologue_folded_in_d20_sampled(dev):
    """The d20 shape: the folded backward against the two-step GPU path (full
    tensors, bf16 bound) and against the oracle chain on sampled heads."""
    import torch
    import causal_self_attention_mha_amd as na
    tr = W.make_train_inputs("d20", seed=21)
    B, T, H = tr.q.shape[:3]
    c, s = tables("rope", T, 0)
    q_raw, k_raw, v, do = (to_device(a, dev) for a in (tr.q_store, tr.k_store, tr.v_store,
                                                       tr.do_store))
    ct, sn = torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)
    qr, kr = na.qk_norm_rope_fwd(q_raw, k_raw, ct, sn)
    o, lse = na.attn_fwd(qr, kr, v)
    dq, dk, dv = na.attn_bwd(qr, kr, v, o, do, lse, rope=(q_raw, k_raw, ct, sn))
    dq2r, dk2r, _ = na.attn_bwd(qr, kr, v, o, do, lse)
    dq2, dk2 = na.qk_norm_rope_bwd(q_raw, k_raw, dq2r, dk2r, ct, sn)
    # the value gate folded in too (v standing in for the gate's output): the
    # same dq, dk, dv, and the separate gate backward's dve, dgate bit for bit
    ve = torch.flip(k_raw, dims=(1,)).contiguous()
    gd = to_device(W.make_gate_logits(B, T, H, seed=22)[1], dev)
    dq3, dk3, dv3, dve3, dg3 = na.attn_bwd(qr, kr, v, o, do, lse, rope=(q_raw, k_raw, ct, sn),
                                           value_gate=(ve, gd))
    dve4, dg4 = na.value_gate_bwd(ve, gd, dv)
    torch.cuda.synchronize()
    assert torch.equal(dq3, dq) and torch.equal(dk3, dk) and torch.equal(dv3, dv)
    assert torch.equal(dve3, dve4) and torch.equal(dg3, dg4)
    assert_close("dq vs two-step", to_host(dq), to_host(dq2), BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dk vs two-step", to_host(dk), to_host(dk2), BF16_REL_L2, BF16_MAX_ABS)
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    for b, h in ((0, 0), (31, 9), (13, 4)):
        xq = tr.q[b:b + 1, :, h:h + 1].astype(np.float64)
        xk = tr.k[b:b + 1, :, h:h + 1].astype(np.float64)
        rq = oracle.qk_norm_rope_forward(xq, c64, s64, EPS)
        rk = oracle.qk_norm_rope_forward(xk, c64, s64, EPS)
        rdq, rdk, _, _ = oracle.backward(rq, rk, tr.v[b:b + 1, :, h:h + 1],
                                         tr.do[b:b + 1, :, h:h + 1])
        assert_close(f"dq[{b},{h}]", to_host(dq[b:b + 1, :, h:h + 1]),
                     oracle.qk_norm_rope_backward(xq, rdq, c64, s64, EPS), BF16_REL_L2,
                     BF16_MAX_ABS)
        assert_close(f"dk[{b},{h}]", to_host(dk[b:b + 1, :, h:h + 1]),
                     oracle.qk_norm_rope_backward(xk, rdk, c64, s64, EPS), BF16_REL_L2,
                     BF16_MAX_ABS)


@pytest.mark.parametrize("B,T,H,Hk,Wn", [(1, 1, 1, 1, None), (2, 96, 2, 2, None),
                                         (2, 300, 4, 2, None), (1, 257, 2, 2, 64),
                                         (3, 130, 6, 3, 40)])
def test_fwd_with_prologue_folded_in(dev, B, T, H, Hk, Wn):
    """na_attn_fwd_rope (the key rows by the prologue kernel, the query rows
    normalised and rotated as the forward loads them) against the oracle chain
    prologue -> attention forward: o, lse, and the rotated heads q_rot, k_rot.
    k_rot is the prologue kernel's own output bit for bit; q_rot is within one
    bf16 step of it (the row's mean square is summed in another order; plus
    2^-16 where the rotation cancels to nearly zero, on rows of RMS 1).  Then
    the folded backward on the folded forward's outputs, against the oracle
    chain's gradients of the raw heads."""
    import torch
    import causal_self_attention_mha_amd as na
    tr = W.make_train_inputs("d20", B=B, T=T, H=H, seed=660 + T)
    kv = lambda a: np.ascontiguousarray(a[:, :, :Hk])  # noqa: E731
    c, s = tables("rope", T, 0)
    q_raw, k_raw = to_device(tr.q_store, dev), to_device(kv(tr.k_store), dev)
    v, do = to_device(kv(tr.v_store), dev), to_device(tr.do_store, dev)
    ct, sn = torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)
    o, lse, qr, kr = na.attn_fwd(q_raw, k_raw, v, window=Wn, rope=(ct, sn))
    qr2, kr2 = na.qk_norm_rope_fwd(q_raw, k_raw, ct, sn)
    dq, dk, dv = na.attn_bwd(qr, kr, v, o, do, lse, window=Wn, rope=(q_raw, k_raw, ct, sn))
    torch.cuda.synchronize()
    assert torch.equal(kr, kr2)
    step = (qr.float() - qr2.float()).abs() - 2.0 ** -7 * qr2.float().abs() - 2.0 ** -16
    assert float(step.max()) <= 0.0
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    xq, xk = tr.q.astype(np.float64), kv(tr.k).astype(np.float64)
    rq = oracle.qk_norm_rope_forward(xq, c64, s64, EPS)
    rk = oracle.qk_norm_rope_forward(xk, c64, s64, EPS)
    ro, rl = oracle.forward(rq, rk, kv(tr.v), window=Wn)
    assert_close("q_rot", to_host(qr), rq, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("k_rot", to_host(kr), rk, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("o", to_host(o), ro, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", to_host(lse), rl, BF16_REL_L2, BF16_MAX_ABS)
    rdq, rdk, rdv, _ = oracle.backward(rq, rk, kv(tr.v), tr.do, window=Wn)
    assert_close("dv", to_host(dv), rdv, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dq", to_host(dq), oracle.qk_norm_rope_backward(xq, rdq, c64, s64, EPS),
                 BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dk", to_host(dk), oracle.qk_norm_rope_backward(xk, rdk, c64, s64, EPS),
                 BF16_REL_L2, BF16_MAX_ABS)


def test_fwd_with_prologue_folded_in_d20_sampled(dev):
    """The d20 shape in the launch the benchmark times: the folded forward
    against the two-step GPU path (prologue kernel, then the forward) on the
    full tensors, and o, lse against the oracle chain on sampled heads."""
    import torch
    import causal_self_attention_mha_amd as na
    tr = W.make_train_inputs("d20", seed=23)
    B, T, H = tr.q.shape[:3]
    c, s = tables("rope", T, 0)
    q_raw, k_raw, v = (to_device(a, dev) for a in (tr.q_store, tr.k_store, tr.v_store))
    ct, sn = torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev)
    o, lse, qr, kr = na.attn_fwd(q_raw, k_raw, v, rope=(ct, sn))
    qr2, kr2 = na.qk_norm_rope_fwd(q_raw, k_raw, ct, sn)
    o2, lse2 = na.attn_fwd(qr2, kr2, v)
    torch.cuda.synchronize()
    assert torch.equal(kr, kr2)
    step = (qr.float() - qr2.float()).abs() - 2.0 ** -7 * qr2.float().abs() - 2.0 ** -16
    assert float(step.max()) <= 0.0
    assert_close("o vs two-step", to_host(o), to_host(o2), BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse vs two-step", to_host(lse), to_host(lse2), BF16_REL_L2, BF16_MAX_ABS)
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    for b, h in ((0, 0), (31, 9), (17, 5)):
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        rq = oracle.qk_norm_rope_forward(tr.q[sl].astype(np.float64), c64, s64, EPS)
        rk = oracle.qk_norm_rope_forward(tr.k[sl].astype(np.float64), c64, s64, EPS)
        ro, rl = oracle.forward(rq, rk, tr.v[sl])
        assert_close(f"o[{b},{h}]", to_host(o[sl]), ro, BF16_REL_L2, BF16_MAX_ABS)
        assert_close(f"lse[{b},{h}]", to_host(lse[b:b + 1, h:h + 1]), rl, BF16_REL_L2,
                     BF16_MAX_ABS)
