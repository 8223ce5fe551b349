"""The seeded input generator: determinism, shapes, bf16 rounding, sinks and samples."""
import numpy as np
import torch

from workloads import get, make
from workloads.synth import bf16_bits_to_f32, f32_to_bf16_bits, position_code


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([1.00390625, 1.01171875, -2.00781250, 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
    assert np.array_equal(bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_position_code_layout():
    pe = position_code((4, 8, 8), 64, (1.0, 1.0, 1.0))
    assert pe.shape == (256, 64)
    # token (t=1, h=0, w=0): t block channel 0 = sin(1), channel 1 = cos(1); h, w blocks at c=0
    n = 1 * 64
    assert np.isclose(pe[n, 0], np.sin(1.0)) and np.isclose(pe[n, 1], np.cos(1.0))
    assert pe[n, 24] == 0.0 and pe[n, 25] == 1.0 and pe[n, 44] == 0.0 and pe[n, 45] == 1.0


def test_tiny_and_small_deterministic():
    a, b = make(get(0)), make(get(0))
    assert np.array_equal(a.q, b.q) and np.array_equal(a.w1, b.w1)
    s = make(get(1), heads=[2])
    full = make(get(1))
    assert np.array_equal(s.q[:, 2], full.q[:, 2]) and np.array_equal(s.k[:, 2], full.k[:, 2])
    assert full.q.dtype == np.uint16 and full.q.shape == (1, 12, 4096, 128)
    assert len(full.sinks) == 4 and full.w1.shape == (12, 384, 256) and full.w2.shape == (12, 256, 64)
    kf = full.head("k", 0, 5)
    qf = full.head("q", 0, 5)
    ratio = np.linalg.norm(kf[full.sinks], axis=1).mean() / np.linalg.norm(kf, axis=1).mean()
    assert ratio > 3.0
    assert abs(np.linalg.norm(qf, axis=1).mean() - np.linalg.norm(np.delete(kf, full.sinks, 0), axis=1).mean()) < 0.5


def test_shapes_and_samples():
    c3 = get(3)
    assert c3.valid_shapes() == [(2, 8, 8), (4, 4, 8), (1, 8, 16)]
    assert get(4).valid_shapes() == [(2, 8, 8), (4, 4, 8), (1, 8, 16), (8, 4, 4)]
    assert get(1).head_shapes()[:4] == [(2, 8, 8), (8, 4, 4), (1, 8, 16), (4, 4, 8)]
    assert c3.n_tiles == 600 and get(4).n_tiles == 1200
    assert abs(c3.kept_flops(60) - 1.2079e13) / 1.2079e13 < 1e-3
