"""CPU checks of the seeded input generators (shared by the oracle checks and
the GPU path): shapes pinned to the figures the pages print, reproducibility,
draw order, and bf16 round-to-nearest-even against torch's own conversion."""
import json
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")


def test_configs_match_page_figures():
    g = json.load(open(GOLDEN, encoding="utf-8"))
    d20 = W.CONFIGS["d20"]
    assert d20.H * d20.D == g["d20"]["channels"]
    assert d20.H == g["d20"]["heads"] and d20.D == g["d20"]["head_dim"]
    assert d20.B == g["device_batch_size_default"]["value"]
    assert W.CONFIGS["d26"].B == g["device_batch_size_d26"]["value"]
    for name in ("d12", "d20", "d26"):
        c = W.CONFIGS[name]
        assert c.T == g["sequence_length"]["value"]
        depth = int(name[1:])
        assert depth in g["depth_dial"]["depths"]
        # width = 64 * depth (d20 -> 1280) at head dim 128
        assert c.H * c.D == 64 * depth, name
    dec = W.CONFIGS["decode_d20"]
    assert dec.H == g["d20"]["heads"] and dec.T_cap == g["sequence_length"]["value"]


def test_bf16_rne_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        (rng.standard_normal(1000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.3895314e38], dtype=np.float32),
    ])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to even: 1 + 2^-8 -> 1.0 ; 1 + 3*2^-8 -> 1 + 2^-6
    t = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8], dtype=np.float32)
    assert list(W.bf16_bits_to_f32(W.f32_to_bf16_bits(t))) == [1.0, 1 + 2.0 ** -6]
    assert W.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_train_inputs_reproducible_and_distributed():
    a = W.make_train_inputs("d20", B=2, T=64, H=3)
    b = W.make_train_inputs("d20", B=2, T=64, H=3)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.do, b.do)):
        assert np.array_equal(x, y)
    assert a.q.shape == (2, 64, 3, 128) and a.q_store.dtype == np.uint16
    assert np.array_equal(W.bf16_bits_to_f32(a.q_store), a.q)
    assert 0.45 < a.q.std() < 0.55 and 0.008 < a.do.std() < 0.012
    # draw order Q, K, V, dO from one PCG64 stream
    rng = np.random.default_rng(W.CONFIGS["d20"].seed)
    q0 = (rng.standard_normal((2, 64, 3, 128)) * 0.5).astype(np.float32)
    assert np.array_equal(W.f32_to_bf16_bits(q0), a.q_store)
    t = W.make_train_inputs("tiny_f32")
    assert t.q.dtype == np.float32 and t.q_store is t.q and t.q.shape == (1, 256, 10, 128)


def test_decode_inputs():
    d = W.make_decode_inputs(B=8, T_cap=300)
    assert d.seqlens.dtype == np.int32 and d.seqlens.min() >= 1 and d.seqlens.max() <= 300
    assert d.k_cache.shape == (8, 300, 10, 128) and d.q.shape == (8, 10, 128)
    full = W.make_decode_inputs()
    assert full.seqlens.shape == (64,)
    rng = np.random.default_rng(W.CONFIGS["decode_d20"].seed)
    assert np.array_equal(full.seqlens, rng.integers(1, 2049, size=64))


def test_prologue_inputs_are_seeded_and_well_formed():
    c1, s1 = W.make_angle_tables(17, 64, seed=3)
    c2, s2 = W.make_angle_tables(17, 64, seed=3)
    assert c1.dtype == np.float32 and c1.shape == (17, 64) and s1.shape == (17, 64)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    # cos^2 + sin^2 = 1 up to the fp32 rounding of each
    assert np.allclose(c1.astype(np.float64) ** 2 + s1.astype(np.float64) ** 2, 1.0, atol=1e-6)
    assert not np.array_equal(W.make_angle_tables(17, 64, seed=4)[0], c1)
    g, bits = W.make_gate_logits(2, 5, 3, seed=7)
    assert g.shape == (2, 5, 3) and bits.dtype == np.uint16
    assert np.array_equal(W.bf16_bits_to_f32(bits), g)      # values are the stored bf16
    assert np.array_equal(W.make_gate_logits(2, 5, 3, seed=7)[1], bits)
