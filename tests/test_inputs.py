"""The seeded input generators: shapes, storage, determinism and the stated laws."""
import numpy as np

from workloads import (CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, normal_f32,
                       zipf_router_bias)
from workloads.generate import cluster_tokens


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                     -2.5, 0.0, -0.0, 3.0e38], np.float32)
    bits = f32_to_bf16_bits(vals)
    back = bf16_bits_to_f32(bits)
    # ties go to the even mantissa; above a tie rounds up
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 4 * 2 ** -8
    assert back[3] == 1.0 + 2 ** -7 and back[4] == -2.5
    assert bits[5] == 0 and bits[6] == 0x8000
    # agrees with torch's own float -> bfloat16 conversion
    import torch
    t = torch.from_numpy(np.random.default_rng(0).standard_normal(10000).astype(np.float32))
    np.testing.assert_array_equal(f32_to_bf16_bits(t.numpy()),
                                  t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_generators_are_deterministic_and_chunk_independent():
    a = normal_f32(0, 3, (3, 1 << 21), 0.5)
    b = normal_f32(0, 3, (3, 1 << 21), 0.5)
    np.testing.assert_array_equal(a, b)
    assert abs(a.std() - 0.5) < 0.01


def test_tiny_config_shapes_and_dtypes():
    cfg = CONFIGS["tiny_fp32"]
    a = make_inputs(cfg)
    assert a["x"].shape == (256, 128) and a["x"].dtype == np.float32
    assert a["W1"].shape == (4, 512, 128) and a["W2"].shape == (4, 128, 512)
    assert a["bg"] is None and a["b1"] is None
    assert abs(a["Wg"].std() - 0.02) < 0.002


def test_zipf_bias_law():
    b = zipf_router_bias(64)
    w = np.exp(2 * b.astype(np.float64))
    assert abs(w.sum() - 1) < 1e-6
    np.testing.assert_allclose(w[0] / w[1], 2 ** 1.1, rtol=1e-5)


def test_cluster_recipe_long_tail():
    x = cluster_tokens(0, 4096, 16)
    # distinct centres: tokens of one cluster sit within noise of each other
    rounded = np.round(x[:, :4], 0)
    _, counts = np.unique(rounded, axis=0, return_counts=True)
    assert counts.max() / 4096 > 0.15          # the top cluster holds about a quarter
