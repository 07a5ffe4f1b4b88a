"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: central finite
differences, closed forms, invariants of softmax attention, an independent
library routine (torch's CPU scaled_dot_product_attention and autograd in
float64) and exact rational arithmetic.  A plausible slip in the oracle — a
dropped scale, a wrong mask direction, a transposed operand, a missing delta
term — fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- gradients

def _loss(q, k, v, do):
    o, _ = oracle.forward(q, k, v)
    return float(np.sum(o * do))


@pytest.mark.parametrize("T,D", [(1, 4), (2, 4), (5, 4), (8, 4), (2, 8), (5, 8), (8, 8)])
def test_finite_differences_all_entries(T, D):
    """Analytic gradients equal central differences of sum(O * dO)."""
    B, H = 1, 2
    q, k, v, do = (rnd((B, T, H, D), s) for s in (1, 2, 3, 4))
    dq, dk, dv, _ = oracle.backward(q, k, v, do)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do)
            x[idx] = old - eps
            lm = _loss(q, k, v, do)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        # relative 1e-6, plus an absolute floor for gradients that vanish
        # (T = 1: dQ and dK are identically zero) where only FD noise is left
        assert np.linalg.norm(fd - g) <= 1e-6 * np.linalg.norm(g) + 1e-8 * math.sqrt(g.size)


def test_finite_differences_sampled_d128():
    """Sampled entries at the real head dim D = 128, T = 16."""
    B, T, H, D = 1, 16, 2, 128
    q, k, v = (rnd((B, T, H, D), s, 0.5) for s in (11, 12, 13))
    do = rnd((B, T, H, D), 14)
    dq, dk, dv, _ = oracle.backward(q, k, v, do)
    rng = np.random.default_rng(15)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do)
            x[idx] = old - eps
            lm = _loss(q, k, v, do)
            x[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(g[idx])), (idx, fd, g[idx])


# ---------------------------------------------------------------- forward closed forms

def test_probabilities_rows_sum_to_one_and_are_causal():
    """With V = I the output is P itself: rows sum to 1, upper triangle 0."""
    T = 24
    Q, K = rnd((T, 32), 21), rnd((T, 32), 22)
    V = np.eye(T, 32)
    O, _ = oracle.forward_head(Q, K, V)
    P = O[:, :T]
    assert np.all(np.abs(P.sum(axis=1) - 1.0) <= 1e-12)
    assert np.all(P[np.triu_indices(T, 1)] == 0.0)
    assert np.all(P >= 0.0)
    P2, _ = oracle.causal_probabilities(Q, K)
    assert np.allclose(P, P2, rtol=0, atol=1e-15)


def test_q_zero_gives_running_mean_and_log_count():
    """Q = 0: every visible score is 0, so P_ij = 1/(i+1), O_i is the mean of
    V_0..V_i and LSE_i = ln(i+1).  Same for K = 0."""
    T, D = 40, 16
    V = rnd((T, D), 31)
    mean = np.cumsum(V, axis=0) / np.arange(1, T + 1)[:, None]
    for Q, K in ((np.zeros((T, D)), rnd((T, D), 32)), (rnd((T, D), 33), np.zeros((T, D)))):
        O, lse = oracle.forward_head(Q, K, V)
        assert np.allclose(O, mean, rtol=0, atol=1e-13)
        if not Q.any():
            assert np.allclose(lse, np.log(np.arange(1, T + 1)), rtol=0, atol=1e-14)


def test_row_zero_and_single_token():
    T, D = 9, 128
    Q, K, V = rnd((T, D), 41), rnd((T, D), 42), rnd((T, D), 43)
    O, lse = oracle.forward_head(Q, K, V)
    assert np.array_equal(O[0], V[0])               # only key 0 is visible
    dot = sum(float(a) * float(b) for a, b in zip(Q[0], K[0]))
    assert abs(lse[0] - dot / math.sqrt(D)) <= 1e-12
    O1, lse1 = oracle.forward_head(Q[:1], K[:1], V[:1])   # T = 1: O = V
    assert np.array_equal(O1, V[:1])


def test_exact_rational_weights():
    """D = 4, so s = 1/2.  With q_i = (2 ln 2, 0, 0, 0) and k_j = (j, ...),
    s q_i.k_j = j ln 2, so the visible weights of row i are 2^j / (2^(i+1) - 1)
    and LSE_i = ln(2^(i+1) - 1).  Expected values are exact rationals."""
    T, D = 6, 4
    Q = np.zeros((T, D))
    Q[:, 0] = 2 * math.log(2.0)
    K = np.zeros((T, D))
    K[:, 0] = np.arange(T)
    K[:, 1:] = rnd((T, D - 1), 51)                  # orthogonal to q: no effect
    Vint = np.random.default_rng(52).integers(-9, 10, size=(T, D))
    O, lse = oracle.forward_head(Q, K, Vint.astype(np.float64))
    for i in range(T):
        den = 2 ** (i + 1) - 1
        for d in range(D):
            exact = Fraction(sum(2 ** j * int(Vint[j, d]) for j in range(i + 1)), den)
            assert abs(O[i, d] - float(exact)) <= 1e-13
        assert abs(lse[i] - math.log(den)) <= 1e-13


def test_constant_and_affine_v():
    T, D = 33, 64
    Q, K = rnd((T, D), 61), rnd((T, D), 62)
    v = rnd((D,), 63)
    O, _ = oracle.forward_head(Q, K, np.tile(v, (T, 1)))
    assert np.allclose(O, np.tile(v, (T, 1)), rtol=0, atol=1e-13)
    V = rnd((T, D), 64)
    a, b = -1.7, rnd((D,), 65)
    O1, _ = oracle.forward_head(Q, K, V)
    O2, _ = oracle.forward_head(Q, K, a * V + b)
    assert np.allclose(O2, a * O1 + b, rtol=0, atol=1e-12)


def test_key_shift_invariance():
    """Adding u to every key shifts row i's scores by s<Q_i,u>: O unchanged,
    LSE_i shifted by exactly that amount."""
    T, D = 30, 128
    Q, K, V = rnd((T, D), 71), rnd((T, D), 72), rnd((T, D), 73)
    u = rnd((D,), 74)
    O1, l1 = oracle.forward_head(Q, K, V)
    O2, l2 = oracle.forward_head(Q, K + u, V)
    assert np.allclose(O1, O2, rtol=0, atol=1e-12)
    assert np.allclose(l2 - l1, (Q @ u) / math.sqrt(D), rtol=0, atol=1e-11)


def test_causal_independence_bitwise():
    """Changing keys and values after position t leaves rows <= t bit-identical."""
    B, T, H, D = 2, 50, 3, 32
    q, k, v = (rnd((B, T, H, D), s) for s in (81, 82, 83))
    o1, l1 = oracle.forward(q, k, v)
    t = 20
    k2, v2 = k.copy(), v.copy()
    k2[:, t + 1:] = rnd(k2[:, t + 1:].shape, 84) * 5
    v2[:, t + 1:] = rnd(v2[:, t + 1:].shape, 85) * 5
    o2, l2 = oracle.forward(q, k2, v2)
    assert np.array_equal(o1[:, :t + 1], o2[:, :t + 1])
    assert np.array_equal(l1[:, :, :t + 1], l2[:, :, :t + 1])
    assert not np.array_equal(o1[:, t + 1:], o2[:, t + 1:])


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("B,T,H,D", [(2, 37, 3, 16), (1, 64, 2, 128), (1, 1, 1, 8)])
def test_against_torch_sdpa_fp64(B, T, H, D):
    """torch's CPU scaled_dot_product_attention (is_causal, default scale
    1/sqrt(D)) and its autograd, in float64: an independent implementation."""
    torch = pytest.importorskip("torch")
    q, k, v, do = (rnd((B, T, H, D), s) for s in (91, 92, 93, 94))
    o, lse = oracle.forward(q, k, v)
    dq, dk, dv, _ = oracle.backward(q, k, v, do)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy(), dtype=torch.float64,
                               requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    to.backward(torch.tensor(do.transpose(0, 2, 1, 3).copy(), dtype=torch.float64))
    back = lambda t: t.detach().numpy().transpose(0, 2, 1, 3)  # noqa: E731
    assert np.allclose(o, back(to), rtol=0, atol=1e-12)
    assert np.allclose(dq, back(tq.grad), rtol=0, atol=1e-11)
    assert np.allclose(dk, back(tk.grad), rtol=0, atol=1e-11)
    assert np.allclose(dv, back(tv.grad), rtol=0, atol=1e-11)
    # LSE: logsumexp of torch-computed masked scores
    S = torch.einsum("bhid,bhjd->bhij", tq.detach(), tk.detach()) / math.sqrt(D)
    S = S.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    assert np.allclose(lse, torch.logsumexp(S, dim=-1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- gradient invariants

def test_gradient_invariants():
    T, D = 45, 128
    Q, K, V, dO = (rnd((T, D), s, 0.7) for s in (101, 102, 103, 104))
    dQ, dK, dV, delta = oracle.backward_head(Q, K, V, dO)
    # rows of P sum to 1  =>  sum_j dV_j = sum_i dO_i
    assert np.allclose(dV.sum(axis=0), dO.sum(axis=0), rtol=0, atol=1e-11)
    # rows of dS sum to 0  =>  sum_j dK_j = 0
    assert np.allclose(dK.sum(axis=0), 0.0, rtol=0, atol=1e-11)
    # query 0 sees one key: its softmax is constant, so dQ_0 = 0
    assert np.allclose(dQ[0], 0.0, rtol=0, atol=1e-14)
    # delta equals rowsum(dO * O) with O from the forward
    O, _ = oracle.forward_head(Q, K, V)
    assert np.allclose(delta, np.sum(dO * O, axis=1), rtol=0, atol=1e-12)


def test_constant_v_kills_q_and_k_gradients():
    T, D = 20, 32
    Q, K, dO = rnd((T, D), 111), rnd((T, D), 112), rnd((T, D), 113)
    V = np.tile(rnd((D,), 114), (T, 1))
    dQ, dK, dV, _ = oracle.backward_head(Q, K, V, dO)
    assert np.allclose(dQ, 0.0, atol=1e-13) and np.allclose(dK, 0.0, atol=1e-13)


def test_q_zero_dv_closed_form():
    """Q = 0: P_ij = 1/(i+1), so dV_j = sum_{i>=j} dO_i / (i+1)."""
    T, D = 25, 16
    K, V, dO = rnd((T, D), 121), rnd((T, D), 122), rnd((T, D), 123)
    _, _, dV, _ = oracle.backward_head(np.zeros((T, D)), K, V, dO)
    w = dO / np.arange(1, T + 1)[:, None]
    expect = np.cumsum(w[::-1], axis=0)[::-1]
    assert np.allclose(dV, expect, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- decode

def test_decode_equals_last_forward_row_and_ignores_tail():
    B, Tc, H, D = 3, 40, 2, 128
    q = rnd((B, H, D), 131, 0.5)
    kc, vc = rnd((B, Tc, H, D), 132, 0.5), rnd((B, Tc, H, D), 133, 0.5)
    lens = np.array([1, 17, 40])
    kp, vp = kc.copy(), vc.copy()
    for b, L in enumerate(lens):          # poison rows the decode must not read
        kp[b, L:] = np.nan
        vp[b, L:] = np.nan
    o, lse = oracle.decode(q, kp, vp, lens)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b, L in enumerate(lens):
        for h in range(H):
            Qf = kc[b, :L, h, :].copy()
            Qf[L - 1] = q[b, h]           # the decoded query is position L-1
            O, l = oracle.forward_head(Qf, kc[b, :L, h, :], vc[b, :L, h, :])
            assert np.allclose(o[b, h], O[L - 1], rtol=0, atol=1e-13)
            assert abs(lse[b, h] - l[L - 1]) <= 1e-13
    # L = 1: o = V_0 and lse = s <q, k_0>
    assert np.array_equal(o[0, 0], vc[0, 0, 0])
    assert abs(lse[0, 1] - np.dot(q[0, 1], kc[0, 0, 1]) / math.sqrt(D)) <= 1e-13


def test_decode_empty_sequence():
    o, l = oracle.decode_head(np.ones(8), np.ones((4, 8)), np.ones((4, 8)), 0)
    assert np.array_equal(o, np.zeros(8)) and l == -np.inf


# ---------------------------------------------------------------- sliding window

def _brute_window_row(q, K, V, i, W):
    """Row i by pure-Python loops over the keys i - W .. i (no numpy matmul)."""
    D = len(q)
    s = 1.0 / math.sqrt(D)
    js = range(max(0, i - W), i + 1)
    z = {j: s * sum(q[d] * K[j][d] for d in range(D)) for j in js}
    m = max(z.values())
    e = {j: math.exp(z[j] - m) for j in js}
    l = sum(e.values())
    o = [sum(e[j] * V[j][d] for j in js) / l for d in range(D)]
    return o, m + math.log(l)


@pytest.mark.parametrize("W", [0, 1, 2, 3, 6, 9])
def test_window_brute_force_loops(W):
    """Each row's softmax over exactly the keys i - W .. i, in plain loops."""
    T, D = 8, 4
    Q, K, V = (rnd((T, D), s) for s in (301, 302, 303))
    O, lse = oracle.forward_head(Q, K, V, window=W)
    for i in range(T):
        o, l = _brute_window_row(Q[i].tolist(), K.tolist(), V.tolist(), i, W)
        assert np.allclose(O[i], o, rtol=0, atol=1e-13)
        assert abs(lse[i] - l) <= 1e-13


def test_window_zero_closed_form():
    """W = 0: every query sees only itself, so O = V, lse = s <q_i, k_i>,
    dV = dO and the one-key softmax has no gradient: dQ = dK = 0."""
    T, D = 11, 16
    Q, K, V, dO = (rnd((T, D), s) for s in (311, 312, 313, 314))
    O, lse = oracle.forward_head(Q, K, V, window=0)
    assert np.array_equal(O, V)
    assert np.allclose(lse, np.sum(Q * K, axis=1) / 4.0, rtol=0, atol=1e-14)
    dQ, dK, dV, delta = oracle.backward_head(Q, K, V, dO, window=0)
    assert np.array_equal(dV, dO)
    assert np.allclose(dQ, 0.0, atol=1e-13) and np.allclose(dK, 0.0, atol=1e-13)
    assert np.allclose(delta, np.sum(dO * V, axis=1), rtol=0, atol=1e-13)


def test_window_covering_the_sequence_is_full_causal():
    B, T, H, D = 1, 13, 2, 8
    q, k, v, do = (rnd((B, T, H, D), s) for s in (321, 322, 323, 324))
    o, lse = oracle.forward(q, k, v)
    dq, dk, dv, _ = oracle.backward(q, k, v, do)
    for W in (T - 1, T, 5 * T):
        ow, lw = oracle.forward(q, k, v, window=W)
        gw = oracle.backward(q, k, v, do, window=W)
        assert np.array_equal(o, ow) and np.array_equal(lse, lw)
        for a, b in zip((dq, dk, dv), gw[:3]):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("T,D,W", [(6, 4, 1), (7, 4, 2), (9, 8, 4)])
def test_window_finite_differences(T, D, W):
    """Banded gradients equal central differences of sum(O * dO)."""
    B, H = 1, 1
    q, k, v, do = (rnd((B, T, H, D), s) for s in (331, 332, 333, 334))
    dq, dk, dv, _ = oracle.backward(q, k, v, do, window=W)
    loss = lambda a, b, c: float(np.sum(oracle.forward(a, b, c, window=W)[0] * do))  # noqa
    eps = 1e-6
    for idx, (x, g) in enumerate(((q, dq), (k, dk), (v, dv))):
        fd = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += eps
            xm[pos] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[idx], args_m[idx] = xp, xm
            fd[pos] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(g, fd, rtol=0, atol=2e-8)


@pytest.mark.parametrize("T,W", [(37, 5), (64, 16), (20, 0)])
def test_window_against_torch_sdpa_fp64(T, W):
    """torch's CPU scaled_dot_product_attention with an explicit boolean band
    mask (allowed iff i - W <= j <= i), and its autograd, in float64."""
    torch = pytest.importorskip("torch")
    B, H, D = 2, 2, 16
    q, k, v, do = (rnd((B, T, H, D), s) for s in (341, 342, 343, 344))
    o, lse = oracle.forward(q, k, v, window=W)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, window=W)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    allowed = (j <= i) & (j >= i - W)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy(), dtype=torch.float64,
                               requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed)
    to.backward(torch.tensor(do.transpose(0, 2, 1, 3).copy(), dtype=torch.float64))
    back = lambda t: t.detach().numpy().transpose(0, 2, 1, 3)  # noqa: E731
    assert np.allclose(o, back(to), rtol=0, atol=1e-12)
    assert np.allclose(dq, back(tq.grad), rtol=0, atol=1e-11)
    assert np.allclose(dk, back(tk.grad), rtol=0, atol=1e-11)
    assert np.allclose(dv, back(tv.grad), rtol=0, atol=1e-11)
    S = torch.matmul(tq.detach(), tk.detach().transpose(-1, -2)) / math.sqrt(D)
    S = S.masked_fill(~allowed, float("-inf"))
    assert np.allclose(lse, torch.logsumexp(S, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_window_decode_equals_last_forward_row_and_ignores_old_keys():
    B, Tc, H, D, W = 3, 40, 2, 32, 7
    q = rnd((B, H, D), 351, 0.5)
    kc, vc = rnd((B, Tc, H, D), 352, 0.5), rnd((B, Tc, H, D), 353, 0.5)
    lens = np.array([1, 8, 40])
    kp, vp = kc.copy(), vc.copy()
    for b, L in enumerate(lens):          # poison rows outside L - 1 - W .. L - 1
        kp[b, L:] = np.nan
        vp[b, L:] = np.nan
        kp[b, :max(0, L - 1 - W)] = np.nan
        vp[b, :max(0, L - 1 - W)] = np.nan
    o, lse = oracle.decode(q, kp, vp, lens, window=W)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b, L in enumerate(lens):
        for h in range(H):
            Qf = kc[b, :L, h, :].copy()
            Qf[L - 1] = q[b, h]
            O, l = oracle.forward_head(Qf, kc[b, :L, h, :], vc[b, :L, h, :], window=W)
            assert np.allclose(o[b, h], O[L - 1], rtol=0, atol=1e-13)
            assert abs(lse[b, h] - l[L - 1]) <= 1e-13


# ---------------------------------------------------------------- grouped-query attention

@pytest.mark.parametrize("H,Hk,W", [(4, 2, None), (6, 2, None), (4, 1, None), (4, 2, 5)])
def test_gqa_against_torch_sdpa_fp64(H, Hk, W):
    """torch's CPU scaled_dot_product_attention(enable_gqa=True) and its
    autograd in float64 (query head h reads key/value head h // (H / Hk))."""
    torch = pytest.importorskip("torch")
    B, T, D = 2, 29, 16
    q, do = rnd((B, T, H, D), 401), rnd((B, T, H, D), 404)
    k, v = rnd((B, T, Hk, D), 402), rnd((B, T, Hk, D), 403)
    o, lse = oracle.forward(q, k, v, window=W)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, window=W)
    assert dk.shape == (B, T, Hk, D)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy(), dtype=torch.float64,
                               requires_grad=True) for x in (q, k, v))
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    allowed = (j <= i) if W is None else (j <= i) & (j >= i - W)
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed,
                                                          enable_gqa=True)
    to.backward(torch.tensor(do.transpose(0, 2, 1, 3).copy(), dtype=torch.float64))
    back = lambda t: t.detach().numpy().transpose(0, 2, 1, 3)  # noqa: E731
    assert np.allclose(o, back(to), rtol=0, atol=1e-12)
    assert np.allclose(dq, back(tq.grad), rtol=0, atol=1e-11)
    assert np.allclose(dk, back(tk.grad), rtol=0, atol=1e-11)
    assert np.allclose(dv, back(tv.grad), rtol=0, atol=1e-11)


def test_gqa_finite_differences():
    B, T, H, Hk, D = 1, 5, 4, 2, 4
    q, do = rnd((B, T, H, D), 411), rnd((B, T, H, D), 414)
    k, v = rnd((B, T, Hk, D), 412), rnd((B, T, Hk, D), 413)
    dq, dk, dv, _ = oracle.backward(q, k, v, do)
    loss = lambda a, b, c: float(np.sum(oracle.forward(a, b, c)[0] * do))  # noqa: E731
    eps = 1e-6
    for idx, (x, g) in enumerate(((q, dq), (k, dk), (v, dv))):
        fd = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += eps
            xm[pos] -= eps
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[idx], args_m[idx] = xp, xm
            fd[pos] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(g, fd, rtol=0, atol=2e-8)


def test_gqa_is_mha_on_repeated_heads():
    """GQA equals MHA with each key/value head repeated for its query heads
    (consecutive query heads share one), and the key/value gradients are the
    group sums of the repeated heads' gradients."""
    B, T, H, Hk, D = 2, 23, 6, 3, 8
    G = H // Hk
    q, do = rnd((B, T, H, D), 421), rnd((B, T, H, D), 424)
    k, v = rnd((B, T, Hk, D), 422), rnd((B, T, Hk, D), 423)
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    o, lse = oracle.forward(q, k, v)
    o2, lse2 = oracle.forward(q, kr, vr)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    dq, dk, dv, _ = oracle.backward(q, k, v, do)
    dq2, dk2, dv2, _ = oracle.backward(q, kr, vr, do)
    assert np.array_equal(dq, dq2)
    assert np.allclose(dk, dk2.reshape(B, T, Hk, G, D).sum(axis=3), rtol=0, atol=1e-13)
    assert np.allclose(dv, dv2.reshape(B, T, Hk, G, D).sum(axis=3), rtol=0, atol=1e-13)
    got = oracle.kv_grads(q, k, v, do, [(1, 2), (0, 0)])
    for (b, hk), (gk, gv) in got.items():
        assert np.allclose(gk, dk[b, :, hk], rtol=0, atol=1e-13)
        assert np.allclose(gv, dv[b, :, hk], rtol=0, atol=1e-13)


def test_gqa_decode_reads_the_group_head():
    B, Tc, H, Hk, D = 2, 30, 4, 2, 16
    q = rnd((B, H, D), 431, 0.5)
    kc, vc = rnd((B, Tc, Hk, D), 432, 0.5), rnd((B, Tc, Hk, D), 433, 0.5)
    lens = np.array([9, 30])
    o, lse = oracle.decode(q, kc, vc, lens)
    for b, L in enumerate(lens):
        for h in range(H):
            Qf = kc[b, :L, h // 2, :].copy()
            Qf[L - 1] = q[b, h]
            O, l = oracle.forward_head(Qf, kc[b, :L, h // 2, :], vc[b, :L, h // 2, :])
            assert np.allclose(o[b, h], O[L - 1], rtol=0, atol=1e-13)
            assert abs(lse[b, h] - l[L - 1]) <= 1e-13


# ---------------------------------------------------------------- prefill over a cache

def _prefill_case(B, T_q, H, Hk, T_cap, lens, seed, D=16):
    q = rnd((B, T_q, H, D), seed)
    kn, vn = rnd((B, T_q, Hk, D), seed + 1), rnd((B, T_q, Hk, D), seed + 2)
    kc, vc = rnd((B, T_cap, Hk, D), seed + 3), rnd((B, T_cap, Hk, D), seed + 4)
    return q, kn, vn, kc, vc, np.array(lens)


def test_prefill_on_an_empty_cache_is_the_forward():
    """L = 0: the chunk attends only to itself, top-left causal = the forward."""
    q, kn, vn, kc, vc, lens = _prefill_case(2, 13, 4, 2, 20, [0, 0], 501)
    o, lse, kc2, vc2 = oracle.prefill(q, kn, vn, kc, vc, lens)
    of, lf = oracle.forward(q, kn, vn)
    assert np.array_equal(o, of) and np.array_equal(lse, lf)
    assert np.array_equal(kc2[:, :13], kn) and np.array_equal(kc2[:, 13:], kc[:, 13:])


def test_prefill_of_one_token_is_decode():
    """T_q = 1: the query at position L sees keys 0 .. L = decode with L + 1 cached rows."""
    q, kn, vn, kc, vc, lens = _prefill_case(3, 1, 4, 2, 30, [0, 7, 29], 511)
    o, lse, kc2, vc2 = oracle.prefill(q, kn, vn, kc, vc, lens)
    od, ld = oracle.decode(q[:, 0], kc2, vc2, lens + 1)
    assert np.allclose(o[:, 0], od, rtol=0, atol=1e-13)
    assert np.allclose(lse[:, :, 0], ld, rtol=0, atol=1e-13)


@pytest.mark.parametrize("W", [None, 0, 3])
def test_prefill_brute_force_loops(W):
    T_q, L, D = 4, 5, 4
    q, kn, vn, kc, vc, _ = _prefill_case(1, T_q, 1, 1, 12, [L], 521, D=D)
    O, lse = oracle.prefill_head(q[0, :, 0], kc[0, :, 0], vc[0, :, 0], kn[0, :, 0], vn[0, :, 0],
                                 L, W)
    K = kc[0, :L, 0].tolist() + kn[0, :, 0].tolist()
    V = vc[0, :L, 0].tolist() + vn[0, :, 0].tolist()
    Wb = 10 ** 9 if W is None else W
    for i in range(T_q):
        o, l = _brute_window_row(q[0, i, 0].tolist(), K, V, L + i, Wb)
        assert np.allclose(O[i], o, rtol=0, atol=1e-13) and abs(lse[i] - l) <= 1e-13


def test_prefill_against_torch_sdpa_fp64():
    """torch's CPU scaled_dot_product_attention with an explicit bottom-right
    causal mask over [cache rows, new rows] and enable_gqa, in float64."""
    torch = pytest.importorskip("torch")
    B, T_q, H, Hk, T_cap, D = 2, 9, 4, 2, 30, 16
    q, kn, vn, kc, vc, lens = _prefill_case(B, T_q, H, Hk, T_cap, [6, 17], 531, D=D)
    o, lse, kc2, vc2 = oracle.prefill(q, kn, vn, kc, vc, lens)
    for b in range(B):
        L = int(lens[b])
        K = torch.tensor(kc2[b, :L + T_q].transpose(1, 0, 2).copy())[None]
        V = torch.tensor(vc2[b, :L + T_q].transpose(1, 0, 2).copy())[None]
        Q = torch.tensor(q[b].transpose(1, 0, 2).copy())[None]
        i = torch.arange(T_q)[:, None]
        j = torch.arange(L + T_q)[None, :]
        to = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=j <= L + i,
                                                              enable_gqa=True)
        assert np.allclose(o[b], to[0].numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- prologue: QK norm + RoPE

def test_prologue_position_zero_is_rms_norm():
    """cos = 1, sin = 0: the output is torch's F.rms_norm (float64, no weight)."""
    torch = pytest.importorskip("torch")
    x = rnd((2, 5, 3, 16), 601)
    c, s = np.ones((5, 8)), np.zeros((5, 8))
    y = oracle.qk_norm_rope_forward(x, c, s, eps=1e-6)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (16,), eps=1e-6).numpy()
    assert np.allclose(y, ref, rtol=0, atol=1e-14)


def test_prologue_rotation_keeps_the_rms_and_shifts_relative_positions():
    """Each row's squared norm is D mean(x^2) / (mean(x^2) + eps); the dot
    product of a rotated query at t1 and key at t2 depends on t1 - t2 only."""
    D, T = 16, 12
    x = rnd((1, T, 1, D), 611)
    c, s = oracle.rope_tables(T, D)
    y = oracle.qk_norm_rope_forward(x, c, s, eps=1e-6)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.sum(y * y, axis=-1), D * ms / (ms + 1e-6), rtol=1e-13, atol=0)
    qv, kv = rnd((D,), 612), rnd((D,), 613)
    Q = oracle.qk_norm_rope_forward(np.tile(qv, (1, T, 1, 1)), c, s)[0, :, 0]
    K = oracle.qk_norm_rope_forward(np.tile(kv, (1, T, 1, 1)), c, s)[0, :, 0]
    for t1, t2, u1, u2 in ((5, 2, 9, 6), (7, 7, 0, 0), (3, 8, 4, 9)):
        assert abs(Q[t1] @ K[t2] - Q[u1] @ K[u2]) < 1e-12


def test_prologue_rotation_angle_closed_form():
    """Dimension pair i of row t turns by theta = t * 10000^(-2 i / D)."""
    D, T = 8, 6
    x = np.zeros((1, T, 1, D))
    x[..., 1] = 1.0                 # z = e_1 * sqrt(D) (up to eps)
    c, s = oracle.rope_tables(T, D)
    y = oracle.qk_norm_rope_forward(x, c, s, eps=0.0)
    th = np.arange(T) * 10000.0 ** (-2.0 / D)
    assert np.allclose(y[0, :, 0, 1], np.sqrt(D) * np.cos(th), atol=1e-13)
    assert np.allclose(y[0, :, 0, 1 + D // 2], np.sqrt(D) * np.sin(th), atol=1e-13)


def test_prologue_backward_finite_differences():
    x, dy = rnd((1, 4, 2, 8), 621), rnd((1, 4, 2, 8), 622)
    c, s = oracle.rope_tables(4, 8)
    g = oracle.qk_norm_rope_backward(x, dy, c, s, eps=1e-6)
    eps = 1e-6
    fd = np.zeros_like(x)
    for pos in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[pos] += eps
        xm[pos] -= eps
        fd[pos] = (np.sum(oracle.qk_norm_rope_forward(xp, c, s) * dy)
                   - np.sum(oracle.qk_norm_rope_forward(xm, c, s) * dy)) / (2 * eps)
    assert np.allclose(g, fd, rtol=0, atol=1e-8)


def test_value_gate_limits_and_midpoint():
    """g -> -inf leaves v; g -> +inf adds 3 ve; g = 0 adds 1.5 ve exactly."""
    v, ve = rnd((2, 3, 2, 8), 631), rnd((2, 3, 2, 8), 632)
    assert np.array_equal(oracle.value_gate_forward(v, ve, np.full((2, 3, 2), -800.0)), v)
    assert np.allclose(oracle.value_gate_forward(v, ve, np.full((2, 3, 2), 800.0)), v + 3 * ve,
                       rtol=0, atol=1e-15)
    assert np.array_equal(oracle.value_gate_forward(v, ve, np.zeros((2, 3, 2))), v + 1.5 * ve)


def test_value_gate_backward_matches_torch_autograd():
    """An independent routine: torch's sigmoid and autograd in float64."""
    torch = pytest.importorskip("torch")
    v, ve = rnd((2, 5, 3, 16), 641), rnd((2, 5, 3, 16), 642)
    g, dy = rnd((2, 5, 3), 643, 2.0), rnd((2, 5, 3, 16), 644)
    tv, tve, tg = (torch.tensor(a, requires_grad=True) for a in (v, ve, g))
    out = tv + 3 * torch.sigmoid(tg).unsqueeze(-1) * tve
    out.backward(torch.tensor(dy))
    assert np.allclose(oracle.value_gate_forward(v, ve, g), out.detach().numpy(), rtol=0,
                       atol=1e-14)
    dve, dg = oracle.value_gate_backward(ve, g, dy)
    assert np.allclose(tv.grad.numpy(), dy)   # dv is dv_out itself
    assert np.allclose(dve, tve.grad.numpy(), rtol=0, atol=1e-14)
    assert np.allclose(dg, tg.grad.numpy(), rtol=0, atol=1e-13)


def test_value_gate_backward_finite_differences():
    ve, g, dy = rnd((1, 3, 2, 4), 651), rnd((1, 3, 2), 652), rnd((1, 3, 2, 4), 653)
    v = rnd((1, 3, 2, 4), 654)
    _, dg = oracle.value_gate_backward(ve, g, dy)
    eps = 1e-6
    for pos in np.ndindex(g.shape):
        gp, gm = g.copy(), g.copy()
        gp[pos] += eps
        gm[pos] -= eps
        fd = (np.sum(oracle.value_gate_forward(v, ve, gp) * dy)
              - np.sum(oracle.value_gate_forward(v, ve, gm) * dy)) / (2 * eps)
        assert abs(fd - dg[pos]) < 1e-8
