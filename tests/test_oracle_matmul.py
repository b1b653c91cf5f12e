"""Pins of the oracle's W4A16 product (NVFP4 weights [N][K], activations [M][K]) against facts fixed
outside it: an independent dequantisation (E2M1 values from the page's table, E4M3 decoded by torch)
multiplied with numpy, identity and one-hot activations (one exact product per output), and zeros."""
import numpy as np
import pytest

import oracle
import synth
from tests import indep


def weights(n, k, seed, mode="4o6"):
    W = synth.normal_bf16(n, k, seed)
    r = oracle.quantize(W, mode, 2 if mode in ("cjso", "soar") else 0)
    return r["codes"], r["scales"], r["alpha"]


def dequant_indep(codes, scales, alpha, n, k):
    q = indep.e2m1_decode(indep.unpack(codes).reshape(n, k))
    d = np.repeat(indep.e4m3_decode(scales.reshape(n, k // 16)), 16, axis=1)
    return q * d * float(np.float32(alpha))  # exact in binary64: 2 + 4 + 24 significant bits


@pytest.mark.parametrize("m,n,k,mode", [(3, 32, 64, "4o6"), (5, 48, 160, "soar"), (1, 16, 1024, "max")])
def test_matches_numpy_product_of_independent_dequantisation(m, n, k, mode):
    codes, scales, alpha = weights(n, k, seed=m + n, mode=mode)
    X = synth.normal_bf16(m, k, seed=7 * m)
    Y = oracle.matmul(X, codes, scales, alpha, n)
    x = indep.as_f32(X).astype(np.float64)
    Wh = dequant_indep(codes, scales, alpha, n, k)
    ref = x @ Wh.T
    bound = k * 2.0 ** -52 * (np.abs(x) @ np.abs(Wh).T) + 1e-300
    assert np.all(np.abs(Y - ref) <= bound)


def test_identity_rows_give_the_dequantised_weights_exactly():
    n, k = 24, 64
    codes, scales, alpha = weights(n, k, seed=3, mode="cjso")
    X = indep.bf16_bits(np.eye(k, dtype=np.float32)) if hasattr(indep, "bf16_bits") else \
        (np.eye(k, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    Y = oracle.matmul(X, codes, scales, alpha, n)
    assert np.array_equal(Y, dequant_indep(codes, scales, alpha, n, k).T)


def test_one_hot_and_zero_activations():
    n, k = 16, 48
    codes, scales, alpha = weights(n, k, seed=5)
    X = np.zeros((2, k), np.float32)
    X[1, 17] = -3.25
    Y = oracle.matmul(X, codes, scales, alpha, n)
    Wh = dequant_indep(codes, scales, alpha, n, k)
    assert np.all(Y[0] == 0.0)
    assert np.array_equal(Y[1], -3.25 * Wh[:, 17])


def test_bad_arguments():
    codes, scales, alpha = weights(16, 32, seed=1)
    with pytest.raises(ValueError):
        oracle.matmul(np.zeros((2, 24), np.float32), codes[:, :12], scales[:, :1], alpha, 16)
