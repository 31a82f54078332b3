"""The seeded synthetic KV generator: shape, determinism and value structure."""

import numpy as np

from kv_cache_compression_layer_amd.synth import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, generate_kv


def test_shape_and_determinism():
    a = generate_kv(3, 40, 2, 8, seed=5, block_tokens=7)
    b = generate_kv(3, 40, 2, 8, seed=5, block_tokens=256)
    assert a.shape == (3, 2, 40, 2, 8) and a.dtype == np.uint16
    np.testing.assert_array_equal(a, b)  # block size does not change the stream
    assert not np.array_equal(a, generate_kv(3, 40, 2, 8, seed=6))


def test_ar1_and_outliers():
    L, T, H, D = 2, 4000, 1, 100
    x = bf16_bits_to_f32(generate_kv(L, T, H, D, rho=0.9, outlier_frac=0.05, outlier_scale=20.0, seed=1))
    x = x.reshape(L, 2, T, H * D).astype(np.float64)
    r1 = np.mean([np.corrcoef(x[0, 0, :-1, c], x[0, 0, 1:, c])[0, 1] for c in range(H * D)])
    assert abs(r1 - 0.9) < 0.02
    std = x[0, 0].std(axis=0)
    assert np.sum(std > 4 * np.median(std)) == 5  # round(0.05 * 100) outlier channels (seeded)


def test_bf16_rounding_ties_to_even():
    v = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -1.5, 0.0], np.float32)
    np.testing.assert_array_equal(bf16_bits_to_f32(f32_to_bf16_bits(v)), [1.0, 1.0 + 2 * 2.0**-7, -1.5, 0.0])


def test_named_workloads():
    w = WORKLOADS["llama31_8b_t32k"]
    assert w.shape == (32, 2, 32768, 8, 128) and w.raw_bytes == 2 * 2**31
    assert WORKLOADS["glm4_9b_t16k"].innovations == "laplace"
