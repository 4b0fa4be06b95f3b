"""Seeded input generator: determinism, bf16 rounding, workload structure (CPU only)."""
import numpy as np
import pytest
import torch

from synth import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(1e3),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, np.inf, -np.inf], dtype=np.float32),
        # exact halfway cases: ties go to even
        (np.arange(1, 2000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32),
    ])
    ours = f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours), torch.from_numpy(a).to(torch.bfloat16).float().numpy())
    nan = f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(bf16_bits_to_f32(nan))[0]


def test_configs_match_workloads():
    c = CONFIGS
    assert (c["tiny"].B, c["tiny"].N, c["tiny"].d, c["tiny"].S, c["tiny"].k, c["tiny"].n_s) == (1, 1000, 64, 64, 3, 16)
    assert (c["base"].B, c["base"].N, c["base"].n_s, c["base"].m_t) == (8, 8192, 32, 1536)
    assert (c["long"].B, c["long"].N, c["long"].n_s, c["long"].n_centroids) == (2, 32768, 128, 128)
    assert (c["extreme"].N, c["extreme"].n_s) == (98304, 384)
    assert (c["wide"].B, c["wide"].N, c["wide"].d, c["wide"].S, c["wide"].k, c["wide"].m_t) == (4, 16384, 1024, 512, 7, 2048)


def test_seeded_determinism_and_layout():
    cfg = CONFIGS["long"].with_(B=2, N=1300, d=64, m_t=96, m=160)
    a, b = make_inputs(cfg), make_inputs(cfg)
    np.testing.assert_array_equal(a.x, b.x)
    np.testing.assert_array_equal(a.P, b.P)
    np.testing.assert_array_equal(a.z, b.z)
    c = make_inputs(cfg, seed=1)
    assert not np.array_equal(a.x, c.x)
    assert a.x.dtype == np.uint16 and a.x.shape == (2, 1300, 64)
    assert a.P.shape == (cfg.S, (cfg.k + 1) * cfg.S)
    head = bf16_bits_to_f32(a.z[..., : cfg.m - cfg.m_t])
    tail = a.z_tail_f64()
    assert np.isnan(head).all() and np.isfinite(tail).all() and (tail >= 0).all()
    assert tail.shape == (2, 1300, 96)


def test_mixture_structure():
    cfg = CONFIGS["long"].with_(B=1, N=4096, d=128, m_t=64, m=64)
    inp = make_inputs(cfg)
    x = inp.x_f64(0)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    cos = u[:512] @ u[:512].T
    # tokens of one centroid are nearly parallel (noise 0.3 per coordinate, d=128); others are not
    assert (cos > 0.85).sum() > 512 * 2 and (np.abs(cos) < 0.5).mean() > 0.8


def test_duplicates_are_exact():
    cfg = CONFIGS["wide"].with_(B=2, N=4096, d=64, S=512, m_t=64, m=128)
    inp = make_inputs(cfg)
    assert len(inp.meta["dups"]) == 4
    for b, s, t in inp.meta["dups"]:
        np.testing.assert_array_equal(inp.x[b, s * 512:(s + 1) * 512], inp.x[b, t * 512:(t + 1) * 512])
        assert len({s, t}) == 2


def test_tiny_is_fp32_relu_squared():
    inp = make_inputs("tiny")
    assert inp.x.dtype == np.float32 and inp.x.shape == (1, 1000, 64)
    np.testing.assert_array_equal(inp.z, np.maximum(inp.x, 0) ** 2)
    a = np.sqrt(6.0 / (256 + 64))
    assert np.abs(inp.P).max() <= a and inp.P.shape == (64, 256)
