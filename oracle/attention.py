"""fp64 CPU oracle for fused causal multi-head self-attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the graft entry's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP kernels
(neither side imports the other); both consume the seeded arrays produced by
the `workloads` module.

What it computes.  nanochat calls attention as
flash_attn_func(q, k, v, causal=True, window_size=...) on (B, T, H, D)
tensors (apidog blog "ChatGPTを50ドルで独自にトレーニングする方法" — "How to train
your own ChatGPT for $50" — section 5 "Flash Attention integration"; the
(B, T, n_kv_head, head_dim) view is in section 1 "GPT model"), and decodes
through flash_attn_with_kvcache over a prefilled prompt cache (same blog,
section 6 "inference engine").  The pages never write the formula out.  The
readings taken here (plainest, all listed in the design notes):

  * scaled dot-product attention, softmax over keys, scale s = 1/sqrt(D);
  * causal = top-left aligned with T_q = T_k: key j visible to query i iff j <= i;
  * full causal window by default (the long "L" layers of the SSSL pattern);
    with a window W (the short "S" layers, same blog, section 1 "GPT model",
    and the window_size argument of section 5), key j is visible to query i
    iff i - W <= j <= i: the query itself and the W keys before it.  The blog
    gives neither W nor the argument's convention; this is flash-attention's
    (left, right) = (W, 0) band under a causal mask;
  * n_kv_head = n_head (plain multi-head attention) by default; with fewer
    key/value heads (GQA, same blog, section 1: fewer KV heads than query
    heads for faster inference), H is a multiple of H_kv and query head h
    reads key/value head h // (H / H_kv), the grouping of torch's
    scaled_dot_product_attention(enable_gqa=True); a key/value head's
    gradient is the sum over the query heads that read it;
  * LSE is the natural log of sum_j exp(s * q_i . k_j) over visible keys;
  * the loss depends on O only, so the LSE output receives no gradient;
  * decode: the single new query is the last cached position and sees all
    L_b cached keys (bottom-right alignment); the cache already holds it;
  * prefill over a cache (the engine's prefilled prompt cache, same blog,
    section 6): a chunk of T_q new tokens of a sequence whose cache holds L
    rows is appended at rows L .. L + T_q - 1, and its query i sits at
    position L + i and sees keys 0 .. L + i (bottom-right causal alignment,
    flash_attn_with_kvcache's convention); with a window W, keys
    L + i - W .. L + i.

Everything is the plain definition in float64, one (batch, head) at a time,
with dense T x T matrices; numpy's matmul is the only library primitive.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "softmax_scale", "forward_head", "backward_head", "forward", "backward",
    "decode_head", "decode", "causal_probabilities", "kv_head", "kv_grads",
    "prefill_head", "prefill",
]


def kv_head(h: int, H: int, H_kv: int) -> int:
    """Key/value head read by query head h (H a multiple of H_kv)."""
    if H % H_kv != 0:
        raise ValueError(f"H={H} is not a multiple of H_kv={H_kv}")
    return h // (H // H_kv)


def softmax_scale(D: int) -> float:
    """s = 1/sqrt(D): the usual scaled-dot-product scale (FlashAttention's
    default when no scale is passed, as in the call the blog shows)."""
    return 1.0 / math.sqrt(D)


def _scores(Q: np.ndarray, K: np.ndarray, window=None) -> np.ndarray:
    """S_ij = s * <Q_i, K_j>, with S_ij = -inf where j > i (causal mask) and,
    given a window W, where j < i - W (the band's lower edge)."""
    T, D = Q.shape
    S = softmax_scale(D) * (Q @ K.T)
    S[np.triu_indices(T, k=1, m=K.shape[0])] = -np.inf
    if window is not None:
        S[np.tril_indices(T, k=-int(window) - 1, m=K.shape[0])] = -np.inf
    return S


def causal_probabilities(Q, K, window=None):
    """P = softmax over keys of the masked scaled scores, and LSE per row.

    Returns (P, lse) with P (T, T) and lse (T,) in float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    S = _scores(Q, K, window)
    m = S.max(axis=1)                     # row max over visible keys (finite: j = i)
    E = np.exp(S - m[:, None])            # masked entries give exp(-inf) = 0
    l = E.sum(axis=1)
    P = E / l[:, None]
    lse = m + np.log(l)
    return P, lse


def forward_head(Q, K, V, window=None):
    """One (batch, head): O = softmax(s Q K^T + causal mask) V and LSE.

    Q, K, V: (T, D).  Returns O (T, D) and lse (T,) in float64.
    """
    P, lse = causal_probabilities(Q, K, window)
    O = P @ np.asarray(V, dtype=np.float64)
    return O, lse


def backward_head(Q, K, V, dO, window=None):
    """Analytic gradients of L = sum(O * dO) for one (batch, head).

    With P the attention probabilities (recomputed here), O = P V:
      dV = P^T dO
      dP = dO V^T
      delta_i = sum_d dO_id O_id          (= sum_j P_ij dP_ij)
      dS = P * (dP - delta)               (softmax Jacobian, row by row)
      dQ = s dS K
      dK = s dS^T Q
    Returns dQ, dK, dV (T, D) and delta (T,), all float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    s = softmax_scale(Q.shape[1])
    P, _ = causal_probabilities(Q, K, window)
    O = P @ V
    dV = P.T @ dO
    dP = dO @ V.T
    delta = np.sum(dO * O, axis=1)
    dS = P * (dP - delta[:, None])
    dQ = s * (dS @ K)
    dK = s * (dS.T @ Q)
    return dQ, dK, dV, delta


def _heads(x):
    """(B, T, H, D) -> iterator over ((b, h), (T, D) float64 slice)."""
    B, T, H, D = x.shape
    for b in range(B):
        for h in range(H):
            yield (b, h), np.asarray(x[b, :, h, :], dtype=np.float64)


def forward(q, k, v, heads=None, window=None):
    """Batched forward over (B, T, H, D) arrays.

    heads: optional iterable of (b, h) pairs; when given, only those heads are
    computed and the result is a dict {(b, h): (O, lse)}.  Otherwise returns
    o (B, T, H, D) and lse (B, H, T) in float64.  window: None (full causal)
    or W >= 0 (see the module notes).
    """
    B, T, H, D = q.shape
    Hk = k.shape[2]
    kh = lambda h: kv_head(h, H, Hk)  # noqa: E731
    if heads is not None:
        return {(b, h): forward_head(q[b, :, h, :], k[b, :, kh(h), :], v[b, :, kh(h), :], window)
                for (b, h) in heads}
    o = np.empty((B, T, H, D), dtype=np.float64)
    lse = np.empty((B, H, T), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            O, L = forward_head(q[b, :, h, :], k[b, :, kh(h), :], v[b, :, kh(h), :], window)
            o[b, :, h, :] = O
            lse[b, h, :] = L
    return o, lse


def backward(q, k, v, do, heads=None, window=None):
    """Batched backward over (B, T, H, D) arrays (k, v: (B, T, H_kv, D)).

    Returns dq (B, T, H, D), dk, dv (B, T, H_kv, D) and delta (B, H, T) in
    float64, or, when `heads` is given, a dict {(b, h): (dQ, dK, dV, delta)}
    for those query heads, where dK and dV are query head h's share of its
    key/value head's gradient (see kv_grads for the group sums).
    """
    B, T, H, D = q.shape
    Hk = k.shape[2]
    kh = lambda h: kv_head(h, H, Hk)  # noqa: E731
    if heads is not None:
        return {(b, h): backward_head(q[b, :, h, :], k[b, :, kh(h), :], v[b, :, kh(h), :],
                                      do[b, :, h, :], window) for (b, h) in heads}
    dq = np.empty((B, T, H, D), dtype=np.float64)
    dk = np.zeros((B, T, Hk, D), dtype=np.float64)
    dv = np.zeros_like(dk)
    delta = np.empty((B, H, T), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            gq, gk, gv, dl = backward_head(q[b, :, h, :], k[b, :, kh(h), :], v[b, :, kh(h), :],
                                           do[b, :, h, :], window)
            dq[b, :, h, :] = gq
            dk[b, :, kh(h), :] += gk
            dv[b, :, kh(h), :] += gv
            delta[b, h, :] = dl
    return dq, dk, dv, delta


def kv_grads(q, k, v, do, kv_heads, window=None):
    """{(b, hk): (dK, dV)} for the listed key/value heads: the sums, over the
    query heads that read head hk, of their backward_head shares."""
    H, Hk = q.shape[2], k.shape[2]
    G = H // Hk
    out = {}
    for (b, hk) in kv_heads:
        dK = np.zeros(k.shape[1:2] + k.shape[3:], dtype=np.float64)
        dV = np.zeros_like(dK)
        for h in range(hk * G, hk * G + G):
            _, gk, gv, _ = backward_head(q[b, :, h, :], k[b, :, hk, :], v[b, :, hk, :],
                                         do[b, :, h, :], window)
            dK += gk
            dV += gv
        out[(b, hk)] = (dK, dV)
    return out


def decode_head(q, K, V, L: int, window=None):
    """Single-query attention over the first L cached keys of one head.

    q: (D,), K, V: (T_cap, D).  z_j = s <q, K_j> for j < L; o = softmax(z) V[:L];
    lse = logsumexp(z).  Rows >= L are never read.  L = 0 gives o = 0 and
    lse = -inf (an empty softmax).  The query sits at position L - 1, so a
    window W keeps keys L - 1 - W .. L - 1 only.
    """
    D = q.shape[0]
    if L <= 0:
        return np.zeros(D), -np.inf
    j0 = 0 if window is None else max(0, L - 1 - int(window))
    q = np.asarray(q, dtype=np.float64)
    Kl = np.asarray(K[j0:L], dtype=np.float64)
    Vl = np.asarray(V[j0:L], dtype=np.float64)
    z = softmax_scale(D) * (Kl @ q)
    m = z.max()
    e = np.exp(z - m)
    l = e.sum()
    return (e / l) @ Vl, m + math.log(l)


def decode(q, k_cache, v_cache, seqlens, pairs=None, window=None):
    """Batched decode.  q (B, H, D); caches (B, T_cap, H_kv, D); seqlens int [B].

    Returns o (B, H, D) and lse (B, H) in float64, or a dict {(b, h): (o, lse)}
    when `pairs` lists the (b, h) pairs to compute.
    """
    B, H, D = q.shape
    Hk = k_cache.shape[2]
    kh = lambda h: kv_head(h, H, Hk)  # noqa: E731
    if pairs is not None:
        return {(b, h): decode_head(q[b, h], k_cache[b, :, kh(h), :], v_cache[b, :, kh(h), :],
                                    int(seqlens[b]), window) for (b, h) in pairs}
    o = np.empty((B, H, D), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            ob, lb = decode_head(q[b, h], k_cache[b, :, kh(h), :], v_cache[b, :, kh(h), :],
                                 int(seqlens[b]), window)
            o[b, h] = ob
            lse[b, h] = lb
    return o, lse


def prefill_head(q, K_cache, V_cache, k_new, v_new, L: int, window=None):
    """One (batch, head) of a prefill over a cache holding L rows.

    q, k_new, v_new: (T_q, D); K_cache, V_cache: (T_cap, D), rows < L valid.
    The keys are K_cache[:L] followed by k_new (likewise the values); query i
    sees keys j <= L + i (and j >= L + i - window).  Returns O (T_q, D) and
    lse (T_q,) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    T_q, D = q.shape
    K = np.concatenate([np.asarray(K_cache[:L], np.float64), np.asarray(k_new, np.float64)])
    V = np.concatenate([np.asarray(V_cache[:L], np.float64), np.asarray(v_new, np.float64)])
    S = softmax_scale(D) * (q @ K.T)                  # (T_q, L + T_q)
    i = np.arange(T_q)[:, None]
    j = np.arange(L + T_q)[None, :]
    hidden = j > L + i
    if window is not None:
        hidden |= j < L + i - int(window)
    S[hidden] = -np.inf
    m = S.max(axis=1)                                 # finite: key L + i is visible
    E = np.exp(S - m[:, None])
    l = E.sum(axis=1)
    return (E / l[:, None]) @ V, m + np.log(l)


def prefill(q, k_new, v_new, k_cache, v_cache, cache_lens, window=None, pairs=None):
    """Batched prefill.  q (B, T_q, H, D); k_new, v_new (B, T_q, H_kv, D);
    caches (B, T_cap, H_kv, D); cache_lens int [B] (rows already cached,
    L_b + T_q <= T_cap).

    Returns o (B, T_q, H, D), lse (B, H, T_q) and the caches after the append
    (new arrays; the inputs are not modified), or, when `pairs` lists (b, h)
    query heads, a dict {(b, h): (O, lse)}.
    """
    B, T_q, H, D = q.shape
    Hk = k_new.shape[2]
    kh = lambda h: kv_head(h, H, Hk)  # noqa: E731
    if pairs is not None:
        return {(b, h): prefill_head(q[b, :, h], k_cache[b, :, kh(h)], v_cache[b, :, kh(h)],
                                     k_new[b, :, kh(h)], v_new[b, :, kh(h)],
                                     int(cache_lens[b]), window) for (b, h) in pairs}
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    o = np.empty((B, T_q, H, D), dtype=np.float64)
    lse = np.empty((B, H, T_q), dtype=np.float64)
    for b in range(B):
        L = int(cache_lens[b])
        for h in range(H):
            O, lv = prefill_head(q[b, :, h], k_cache[b, :, kh(h)], v_cache[b, :, kh(h)],
                                 k_new[b, :, kh(h)], v_new[b, :, kh(h)], L, window)
            o[b, :, h] = O
            lse[b, h] = lv
        kc[b, L:L + T_q] = k_new[b]
        vc[b, L:L + T_q] = v_new[b]
    return o, lse, kc, vc
