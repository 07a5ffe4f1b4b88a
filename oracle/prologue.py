"""fp64 CPU oracle for the attention prologue: QK normalisation and rotary
position embedding of the query and key heads.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py): only the tests, the graft
entry's smoke check and the benchmark's CPU-baseline leg may use it.

What it computes.  The nanochat model normalises its query and key heads (QK
norm) and rotates them by position (rotary embedding, RoPE) before attention
(apidog blog "ChatGPTを50ドルで独自にトレーニングする方法", section 1 "GPT
model", architecture features).  The blog gives neither formula; the readings
taken here are the plainest ones:

  * QK normalisation: RMS normalisation of each head vector over its D
    elements, no learned scale, z = x / sqrt(mean(x^2) + eps), eps = 1e-6;
  * rotary embedding (RoFormer's rotation of dimension pairs by a
    position-dependent angle) with the pairs (i, i + D/2), rotated by +theta:
    y_i = z_i cos - z_{i+D/2} sin, y_{i+D/2} = z_i sin + z_{i+D/2} cos, with
    cos, sin tables of shape (T, D/2) passed in (theta_{t,i} =
    t * base^(-2 i / D) with base 10000 in the tests and the benchmark);
  * the rotation keeps the RMS, so normalising before or after it is the same.

The value-embedding gate (ResFormer value residual, same blog and section,
"value embeddings"): on the layers that carry one, a learned value embedding
ve of each key/value head is mixed into v with a per-head gate that depends
on the input: v' = v + 3 sigmoid(g) ve, where g (B, T, H_kv) is the output
of the small ve_gate projection of the first input channels (that projection
is an ordinary matrix product upstream; the gate logits g are taken as an
input here).

Plain float64 numpy, one formula per step.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rope_tables", "qk_norm_rope_forward", "qk_norm_rope_backward",
           "value_gate_forward", "value_gate_backward"]


def rope_tables(T: int, D: int, base: float = 10000.0, pos0: int = 0):
    """cos, sin (T, D/2) of theta_{t,i} = (pos0 + t) * base^(-2 i / D)."""
    i = np.arange(D // 2, dtype=np.float64)
    theta = (pos0 + np.arange(T, dtype=np.float64))[:, None] * base ** (-2.0 * i / D)[None, :]
    return np.cos(theta), np.sin(theta)


def _norm(x, eps):
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r, r


def qk_norm_rope_forward(x, cos, sin, eps: float = 1e-6):
    """x (B, T, H, D); cos, sin (T, D/2).  Returns y (B, T, H, D) float64."""
    D = x.shape[-1]
    z, _ = _norm(x, eps)
    c = np.asarray(cos, np.float64)[None, :, None, :]
    s = np.asarray(sin, np.float64)[None, :, None, :]
    z1, z2 = z[..., :D // 2], z[..., D // 2:]
    return np.concatenate([z1 * c - z2 * s, z1 * s + z2 * c], axis=-1)


def qk_norm_rope_backward(x, dy, cos, sin, eps: float = 1e-6):
    """Gradient of sum(y * dy) with respect to x (the rotation's transpose,
    then the normalisation's Jacobian): dz = R^T dy,
    dx = r (dz - z mean(dz * z)) with r = 1 / sqrt(mean(x^2) + eps)."""
    D = x.shape[-1]
    z, r = _norm(x, eps)
    dy = np.asarray(dy, np.float64)
    c = np.asarray(cos, np.float64)[None, :, None, :]
    s = np.asarray(sin, np.float64)[None, :, None, :]
    d1, d2 = dy[..., :D // 2], dy[..., D // 2:]
    dz = np.concatenate([d1 * c + d2 * s, -d1 * s + d2 * c], axis=-1)
    return r * (dz - z * np.mean(dz * z, axis=-1, keepdims=True))


def _sigmoid(g):
    return 1.0 / (1.0 + np.exp(-np.asarray(g, dtype=np.float64)))


def value_gate_forward(v, ve, g):
    """v, ve (B, T, H_kv, D); g (B, T, H_kv).  v + 3 sigmoid(g) ve, float64."""
    return np.asarray(v, np.float64) + 3.0 * _sigmoid(g)[..., None] * np.asarray(ve, np.float64)


def value_gate_backward(ve, g, dv_out):
    """Gradients of sum(v' * dv_out): dv = dv_out, dve = 3 sigmoid(g) dv_out,
    dg = 3 sigmoid(g) (1 - sigmoid(g)) <ve, dv_out> over D.  Returns
    (dve, dg)."""
    sg = _sigmoid(g)
    dv_out = np.asarray(dv_out, np.float64)
    dve = 3.0 * sg[..., None] * dv_out
    dg = 3.0 * sg * (1.0 - sg) * np.sum(np.asarray(ve, np.float64) * dv_out, axis=-1)
    return dve, dg
