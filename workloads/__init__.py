"""Seeded synthetic inputs for the causal self-attention hot path.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic, and it is the one piece of code
that the fp64 oracle checks and the GPU path both consume: every test and
benchmark gets its Q, K, V, dO and decode lengths from here, so both sides
see bit-identical inputs.

Shapes follow the nanochat pages:
  * head dim 128 and d20 = 1280 channels = 10 heads x 128 (aisight.pl article
    "Karpathy udostepnia nanochat ...", section "Model i zalozenia skalowania");
  * device_batch_size 32, halved to 16 for d26 (GeekNews summary, sections on
    bigger models and on the compute environment);
  * sequence length 2048 (apidog blog "ChatGPTを50ドルで独自にトレーニングする方法",
    section 4 "data loading");
  * (B, T, H, D) layout of q, k, v (same blog, section 1 "GPT model", the
    value-embedding snippet that views a tensor as (B, T, n_kv_head, head_dim)).

Recipe (identical for every consumer):
  rng = numpy.random.default_rng(seed)  (PCG64)
  draw order: decode lengths (decode configs only), then Q, K, V, dO
  each tensor: rng.standard_normal(shape) in float64, times the config's
  scale, rounded to float32, then (bf16 configs) rounded to bfloat16 with
  round-to-nearest-even.  Decode lengths: rng.integers(1, T_cap + 1, size=B).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Config", "CONFIGS", "HEADLINE", "DECODE",
    "f32_to_bf16_bits", "bf16_bits_to_f32",
    "TrainInputs", "DecodeInputs", "make_train_inputs", "make_decode_inputs",
    "make_angle_tables", "make_gate_logits",
]


@dataclass(frozen=True)
class Config:
    name: str
    kind: str            # "train" (fwd + bwd) or "decode" (fwd only, KV cache)
    B: int
    H: int
    D: int
    dtype: str           # "f32" or "bf16"
    seed: int
    qkv_scale: float
    do_scale: float = 0.0
    T: int = 0           # train sequence length
    T_cap: int = 0       # decode cache capacity
    note: str = ""


CONFIGS: dict[str, Config] = {
    c.name: c for c in [
        Config("tiny_f32", "train", B=1, T=256, H=10, D=128, dtype="f32", seed=1,
               qkv_scale=1.0, do_scale=1.0,
               note="d20 heads at a short sequence, fp32, correctness only"),
        Config("d12", "train", B=16, T=2048, H=6, D=128, dtype="bf16", seed=2,
               qkv_scale=0.5, do_scale=1e-2, note="depth 12: width 768 = 6 x 128"),
        Config("d20", "train", B=32, T=2048, H=10, D=128, dtype="bf16", seed=3,
               qkv_scale=0.5, do_scale=1e-2,
               note="depth 20: width 1280 = 10 x 128, device batch 32"),
        Config("d26", "train", B=16, T=2048, H=13, D=128, dtype="bf16", seed=4,
               qkv_scale=0.5, do_scale=1e-2,
               note="depth 26: width 1664 = 13 x 128, device batch halved to 16"),
        Config("decode_d20", "decode", B=64, H=10, D=128, dtype="bf16", seed=5,
               qkv_scale=0.5, T_cap=2048,
               note="d20 chat decode: 64 single-token queries, ragged cache"),
    ]
}
HEADLINE = "d20"
DECODE = "decode_d20"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaN maps to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng: np.random.Generator, shape, scale: float, dtype: str):
    """One tensor: fp64 normal * scale -> fp32 -> (bf16).

    Returns (values_f32, storage) where storage is float32 for "f32" and the
    uint16 bf16 bit pattern for "bf16"; values_f32 is exactly what storage
    holds, widened to float32.
    """
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    if dtype == "f32":
        return x, x
    bits = f32_to_bf16_bits(x)
    return bf16_bits_to_f32(bits), bits


@dataclass
class TrainInputs:
    cfg: Config
    shape: tuple
    # float32 views of the exact stored values (what the oracle consumes)
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    # storage arrays (float32 or uint16 bf16 bits) handed to the device
    q_store: np.ndarray = field(repr=False, default=None)
    k_store: np.ndarray = field(repr=False, default=None)
    v_store: np.ndarray = field(repr=False, default=None)
    do_store: np.ndarray = field(repr=False, default=None)


@dataclass
class DecodeInputs:
    cfg: Config
    seqlens: np.ndarray      # int32 [B], each in [1, T_cap]
    q: np.ndarray            # (B, H, D) float32 values
    k_cache: np.ndarray      # (B, T_cap, H, D) float32 values
    v_cache: np.ndarray
    q_store: np.ndarray = field(repr=False, default=None)
    k_store: np.ndarray = field(repr=False, default=None)
    v_store: np.ndarray = field(repr=False, default=None)


def make_train_inputs(cfg: Config | str, *, B: int | None = None, T: int | None = None,
                      H: int | None = None, seed: int | None = None) -> TrainInputs:
    """Q, K, V, dO for a training config; shape overrides make smaller cases
    with the same value distributions."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if cfg.kind != "train":
        raise ValueError(f"{cfg.name} is not a training config")
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    H = cfg.H if H is None else H
    seed = cfg.seed if seed is None else seed
    shape = (B, T, H, cfg.D)
    rng = np.random.default_rng(seed)
    q, qs = _draw(rng, shape, cfg.qkv_scale, cfg.dtype)
    k, ks = _draw(rng, shape, cfg.qkv_scale, cfg.dtype)
    v, vs = _draw(rng, shape, cfg.qkv_scale, cfg.dtype)
    do, dos = _draw(rng, shape, cfg.do_scale, cfg.dtype)
    return TrainInputs(cfg, shape, q, k, v, do, qs, ks, vs, dos)


def make_decode_inputs(cfg: Config | str = DECODE, *, B: int | None = None,
                       T_cap: int | None = None, H: int | None = None,
                       seed: int | None = None, seqlens=None) -> DecodeInputs:
    """Single-token queries and a padded (B, T_cap, H, D) cache with ragged
    per-sequence lengths drawn uniformly from [1, T_cap]."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if cfg.kind != "decode":
        raise ValueError(f"{cfg.name} is not a decode config")
    B = cfg.B if B is None else B
    T_cap = cfg.T_cap if T_cap is None else T_cap
    H = cfg.H if H is None else H
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, T_cap + 1, size=B).astype(np.int32)
    if seqlens is not None:
        lens = np.asarray(seqlens, dtype=np.int32).copy()
    q, qs = _draw(rng, (B, H, cfg.D), cfg.qkv_scale, cfg.dtype)
    k, ks = _draw(rng, (B, T_cap, H, cfg.D), cfg.qkv_scale, cfg.dtype)
    v, vs = _draw(rng, (B, T_cap, H, cfg.D), cfg.qkv_scale, cfg.dtype)
    return DecodeInputs(cfg, lens, q, k, v, qs, ks, vs)


def make_angle_tables(T_tab: int, half: int = 64, seed: int = 0):
    """cos and sin (T_tab, half) float32 of angles drawn uniformly from
    [-pi, pi): arbitrary rotation tables for the QK-norm + rotary prologue,
    whose kernels take the tables as inputs.  Returns (cos, sin) float32."""
    rng = np.random.default_rng(seed)
    a = rng.uniform(-np.pi, np.pi, size=(T_tab, half))
    return np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)


def make_gate_logits(B: int, T: int, H: int, seed: int = 0, scale: float = 2.0):
    """Per-head gate logits (B, T, H) for the value-embedding gate:
    standard normal * scale, rounded to bf16.  Returns (values_f32, bf16 bits)."""
    return _draw(np.random.default_rng(seed), (B, T, H), scale, "bf16")
