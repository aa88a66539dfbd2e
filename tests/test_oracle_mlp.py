"""Pins for the oracle's linear layers (GPU Pipeline Phase 2b, Kernel
Components 1 matvec convention; PPO CUDA Pipeline Design, Phase A steps 3, 5
and 9) in fp32, bf16-input/fp32-accumulate and the fp64 diagnostic mode."""
import numpy as np
import pytest

import oracle
import synthdata


@pytest.mark.parametrize("dims", [(54, 128), (128, 64), (64, 45), (54, 512), (512, 384),
                                  (384, 256), (64, 1), (99, 128), (128, 51)])
def test_linear_vs_fp64(dims):
    g = np.random.default_rng(sum(dims))
    i, o = dims
    W = (g.standard_normal((o, i)) * np.sqrt(2 / i)).astype(np.float32)
    b = g.standard_normal(o).astype(np.float32)
    x = (g.standard_normal(i) * 2).astype(np.float32)
    ref = W.astype(np.float64) @ x.astype(np.float64) + b
    y = oracle.linear(W, b, x, relu=False)
    scale = np.abs(W.astype(np.float64)) @ np.abs(x.astype(np.float64)) + np.abs(b)
    assert np.all(np.abs(y - ref) <= 1e-6 * scale + 1e-7)
    yr = oracle.linear(W, b, x, relu=True)
    np.testing.assert_array_equal(yr, np.where(y > 0, y, 0))
    y64 = oracle.linear(W, b, x, relu=False, precision=oracle.FP64)
    np.testing.assert_array_equal(y64, ref.astype(np.float32))


def test_zero_weights_give_bias():
    b = np.linspace(-2, 2, 17).astype(np.float32)
    y = oracle.linear(np.zeros((17, 30), np.float32), b, np.ones(30, np.float32), relu=False)
    np.testing.assert_array_equal(y, b)
    y = oracle.linear(np.zeros((17, 30), np.float32), b, np.ones(30, np.float32), relu=True)
    np.testing.assert_array_equal(y, np.maximum(b, 0))


def test_bf16_round_is_rne():
    import struct

    def bits(f):
        return struct.unpack("<I", struct.pack("<f", f))[0]

    def from_bits(u):
        return struct.unpack("<f", struct.pack("<I", u))[0]

    # exactly half way: ties to even
    assert bits(oracle.bf16_round(from_bits(0x3F808000))) == 0x3F800000
    assert bits(oracle.bf16_round(from_bits(0x3F818000))) == 0x3F820000
    assert bits(oracle.bf16_round(from_bits(0x3F808001))) == 0x3F810000
    assert bits(oracle.bf16_round(1.0)) == 0x3F800000
    g = np.random.default_rng(0)
    x = g.standard_normal(10000).astype(np.float32)
    r = np.array([oracle.bf16_round(float(v)) for v in x], np.float32)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0**-8)


def test_bf16_layer_is_exact_products_fp32_sum():
    g = np.random.default_rng(1)
    W = np.array([[oracle.bf16_round(v) for v in row] for row in g.standard_normal((8, 40))],
                 np.float32)
    b = g.standard_normal(8).astype(np.float32)
    x = g.standard_normal(40).astype(np.float32)
    xb = np.array([oracle.bf16_round(v) for v in x], np.float64)
    ref = W.astype(np.float64) @ xb + b
    y = oracle.linear(W, b, x, relu=False, precision=oracle.BF16)
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)


def test_onehot_dense_equals_column_gather():
    """Curiosity layer 1 on [state, onehot(a)]: the dense 99-wide product equals
    the 54-wide product plus column 54+a (fp64 reference)."""
    w = synthdata.ppo_weights(3, bias_scale=0.1)["curiosity"]
    W1, b1 = w[0], w[1]
    g = np.random.default_rng(2)
    for a in range(45):
        s = g.standard_normal(54).astype(np.float32)
        x = np.concatenate([s, np.eye(45, dtype=np.float32)[a]])
        y = oracle.linear(W1, b1, x, relu=False)
        ref = W1[:, :54].astype(np.float64) @ s + W1[:, 54 + a] + b1
        np.testing.assert_allclose(y, ref, rtol=1e-5, atol=1e-5)
