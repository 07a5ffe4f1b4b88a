"""GPU parity at long sequences, beyond the training shapes: T = 32768 for the
forward and backward, a 65536-row cache for decode.

The fp64 oracle computes whole (T, T) score matrices, so at this length it
checks what it can one piece at a time:
  * the first 512 query rows of a random problem: by causality their o, lse
    and dq depend only on the first 512 keys, so the oracle runs on that
    prefix;
  * every row of a problem with K = 0, where attention is uniform over the
    visible keys and the results have closed forms at any length (the
    oracle's own pins check the same forms):
      o_i = mean(V_0 .. V_i),  lse_i = ln(i + 1),  dq = 0,
      dv_j = sum_{i >= j} dO_i / (i + 1),
      dk_j = s sum_{i >= j} (dO_i . V_j - delta_i) q_i / (i + 1),
    with delta_i = dO_i . o_i (dk on sampled rows: each takes O(T D));
  * decode rows one sequence at a time.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import BF16_MAX_ABS, BF16_REL_L2, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu

T_LONG = 32768


def run_train(q_st, k_st, v_st, do_st, dev):
    import torch
    import causal_self_attention_mha_amd as na
    q, k, v, do = (to_device(x, dev) for x in (q_st, k_st, v_st, do_st))
    o, lse = na.attn_fwd(q, k, v)
    dq, dk, dv = na.attn_bwd(q, k, v, o, do, lse)
    torch.cuda.synchronize()
    return {n: to_host(t) for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk),
                                       ("dv", dv))}


def test_long_sequence_prefix_rows(dev):
    inp = W.make_train_inputs("d20", B=1, T=T_LONG, H=2, seed=321)
    got = run_train(inp.q_store, inp.k_store, inp.v_store, inp.do_store, dev)
    for n in ("o", "dq", "dk", "dv"):
        assert np.all(np.isfinite(got[n])), n
    P = 512
    sl = lambda a: np.ascontiguousarray(a[:, :P])  # noqa: E731
    ro, rl = oracle.forward(sl(inp.q), sl(inp.k), sl(inp.v))
    rdq, _, _, _ = oracle.backward(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.do))
    assert_close("o[:512]", got["o"][:, :P], ro, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse[:512]", got["lse"][:, :, :P], rl, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("dq[:512]", got["dq"][:, :P], rdq, BF16_REL_L2, BF16_MAX_ABS)


def test_long_sequence_uniform_attention_closed_forms(dev):
    inp = W.make_train_inputs("d20", B=1, T=T_LONG, H=2, seed=322)
    k_st = np.zeros_like(inp.k_store)
    got = run_train(inp.q_store, k_st, inp.v_store, inp.do_store, dev)
    T, H, D = T_LONG, 2, 128
    s = 1.0 / np.sqrt(D)
    q, v, do = (a[0].astype(np.float64) for a in (inp.q, inp.v, inp.do))  # (T, H, D)
    n = np.arange(1, T + 1, dtype=np.float64)
    o = np.cumsum(v, axis=0) / n[:, None, None]
    assert_close("o", got["o"][0], o, BF16_REL_L2, BF16_MAX_ABS)
    assert_close("lse", got["lse"][0], np.broadcast_to(np.log(n), (H, T)), BF16_REL_L2,
                 BF16_MAX_ABS)
    assert np.all(got["dq"] == 0.0)
    w = 1.0 / n
    dv = np.cumsum((do * w[:, None, None])[::-1], axis=0)[::-1]
    assert_close("dv", got["dv"][0], dv, BF16_REL_L2, BF16_MAX_ABS)
    delta = np.einsum("thd,thd->th", do, o)
    rng = np.random.default_rng(9)
    rows = np.concatenate([[0, 1, 63, 64, 4095, T // 2, T - 65, T - 2, T - 1],
                           rng.integers(0, T, 23)])
    dk_ref = np.zeros((len(rows), H, D))
    for r, j in enumerate(rows):
        a = np.einsum("thd,hd->th", do[j:], v[j]) - delta[j:]          # dP_ij - delta_i
        dk_ref[r] = s * np.einsum("t,th,thd->hd", w[j:], a, q[j:])
    assert_close("dk rows", got["dk"][0][rows], dk_ref, BF16_REL_L2, BF16_MAX_ABS)


def test_decode_long_cache(dev):
    import torch
    import causal_self_attention_mha_amd as na
    lens = [65536, 40001, 1]
    inp = W.make_decode_inputs(B=3, T_cap=65536, H=4, seed=323, seqlens=lens)
    q, kc, vc = (to_device(x, dev) for x in (inp.q_store, inp.k_store, inp.v_store))
    kc[1, 40001:] = float("nan")
    vc[1, 40001:] = float("nan")
    o, lse = na.attn_decode(q, kc, vc, torch.tensor(lens, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    ro, rl = oracle.decode(inp.q, inp.k_cache, inp.v_cache, inp.seqlens)
    go, gl = to_host(o), to_host(lse)
    for b in range(3):  # one at a time: o of the 1-row sequence is far larger
        assert_close(f"o[{b}]", go[b], ro[b], BF16_REL_L2, BF16_MAX_ABS)
        assert_close(f"lse[{b}]", gl[b], rl[b], BF16_REL_L2, BF16_MAX_ABS)
