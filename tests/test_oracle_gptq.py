"""Pins of the GPTQ oracle (oracle/gptq.py) against what GPTQ and the format fix, computed here
independently of the oracle's column loop:
* after the first j columns are fixed at their quantised values, GPTQ's update leaves the later
  weights at the minimiser of the H-weighted error (w - v) H (w - v)^T, a linear solve on H's blocks;
  so the value column j is quantised from is the first entry of that minimiser;
* each code is the nearest E2M1 value of that target over the frozen block scale (brute force);
* with a diagonal H nothing propagates: the codes are plain nearest rounding;
* the damping and dead-input rules, rows computed alone, and the point of GPTQ (a lower H-weighted
  error than plain rounding on correlated inputs)."""
import numpy as np
import pytest

import oracle
import synth
from oracle import gptq as og
from tests import indep

MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def nearest_code(x: np.ndarray) -> np.ndarray:
    """Nearest E2M1 value to binary64 x by exhaustive comparison, ties to the even code."""
    x = np.asarray(x, np.float64).reshape(-1)
    d = np.abs(np.abs(x)[:, None] - MAGS[None, :])
    best = d.min(axis=1)
    cand = d == best[:, None]
    idx = cand.argmax(axis=1)
    idx = np.where((cand.sum(axis=1) == 2) & (idx % 2 == 1), idx + 1, idx)
    return (idx | np.where((x < 0) & (idx > 0), 8, 0)).astype(np.uint8)


def scale_values(scales, alpha):
    d = indep.e4m3_decode(scales).astype(np.float32)
    return (np.float32(alpha) * d).astype(np.float64)


def dequant(codes_unpacked, s_cols):
    mag = MAGS[codes_unpacked & 7]
    return np.where(codes_unpacked & 8, -mag, mag) * s_cols


def prepared(H, percdamp):
    """The damping and dead-input rules, written out here."""
    H = H.copy()
    K = H.shape[0]
    dead = [j for j in range(K) if H[j, j] == 0.0]
    for j in dead:
        H[j, j] = 1.0
    lam = percdamp * sum(H[j, j] for j in range(K)) / K
    for j in range(K):
        H[j, j] += lam
    return H, dead


@pytest.mark.parametrize("R,K,seed,dead,f32", [(5, 48, 1, 0, False), (3, 64, 2, 4, False), (4, 32, 3, 0, False),
                                               (4, 48, 11, 2, True)])
def test_targets_are_the_conditional_optimum(R, K, seed, dead, f32):
    W = synth.normal_f32(R, K, seed) if f32 else synth.normal_bf16(R, K, seed)
    H = synth.hessian(K, seed, dead=dead)
    o = og.gptq(W, H, 0.01, trace=True)
    Hd, dead_cols = prepared(H, 0.01)
    w = indep.as_f32(W).astype(np.float64)
    w[:, dead_cols] = 0.0
    s_cols = np.repeat(scale_values(o["scales"], o["alpha"]), 16, axis=1)
    q = dequant(indep.unpack(o["codes"]), s_cols)
    for j in range(K):
        # v = w_b + (w_a - q_a) H_ab H_bb^-1 minimises the error with columns a = [0, j) fixed
        ea = w[:, :j] - q[:, :j]
        v = w[:, j:] + np.linalg.solve(Hd[j:, j:], (ea @ Hd[:j, j:]).T).T
        np.testing.assert_allclose(o["target"][:, j], v[:, 0], rtol=1e-9, atol=1e-12 * np.abs(w).max())


@pytest.mark.parametrize("R,K,seed", [(16, 128, 4), (6, 256, 5)])
def test_codes_are_nearest_of_their_targets(R, K, seed):
    W = synth.normal_bf16(R, K, seed)
    o = og.gptq(W, synth.hessian(K, seed), trace=True)
    s_cols = np.repeat(scale_values(o["scales"], o["alpha"]), 16, axis=1)
    codes = indep.unpack(o["codes"])
    live = s_cols > 0
    x = o["target"][live] / s_cols[live]
    assert np.array_equal(codes[live], nearest_code(x))
    assert not codes[~live].any()
    assert np.array_equal(o["codes"][:, 0] & 15, codes[:, 0]) and np.array_equal(o["codes"][:, 0] >> 4, codes[:, 1])


def test_diagonal_hessian_is_plain_rounding():
    R, K = 12, 96
    W = synth.normal_bf16(R, K, 6)
    H = np.diag(np.exp2(synth.rng(6).uniform(-3, 3, K)))
    o = og.gptq(W, H, 0.01)
    frame = oracle.quantize(W, "4o6")
    assert np.array_equal(o["scales"], frame["scales"]) and o["alpha"] == frame["alpha"]
    s_cols = np.repeat(scale_values(frame["scales"], frame["alpha"]), 16, axis=1)
    x = indep.as_f32(W).astype(np.float64) / s_cols
    assert np.array_equal(indep.unpack(o["codes"]).reshape(-1), nearest_code(x))


def test_damping_is_a_fraction_of_the_mean_diagonal():
    R, K = 6, 64
    W = synth.normal_bf16(R, K, 7)
    H = synth.hessian(K, 7)
    Hd, _ = prepared(H, 0.05)
    a = og.gptq(W, H, 0.05, trace=True)
    b = og.gptq(W, Hd, 0.0, trace=True)
    np.testing.assert_allclose(a["target"], b["target"], rtol=1e-12, atol=1e-15)
    assert np.array_equal(a["codes"], b["codes"])


def test_dead_inputs_quantise_to_zero():
    R, K = 8, 64
    W = synth.normal_bf16(R, K, 8)
    H = synth.hessian(K, 8, dead=5)
    dead = np.flatnonzero(np.diag(H) == 0.0)
    assert dead.size == 5
    codes = indep.unpack(og.gptq(W, H)["codes"])
    assert not codes[:, dead].any()


def test_rows_alone_equal_the_full_sweep():
    W = synth.normal_bf16(20, 96, 9)
    H = synth.hessian(96, 9)
    full = og.gptq(W, H)
    rows = np.array([0, 7, 19, 3])
    part = og.gptq(W, H, rows=rows)
    assert np.array_equal(part["codes"], full["codes"][rows])


def test_gptq_lowers_the_weighted_error():
    """GPTQ's purpose: on correlated inputs its H-weighted error is well below plain rounding's with
    the same scales (a dropped or mis-signed update loses this)."""
    R, K = 64, 256
    W = synth.normal_bf16(R, K, 10)
    H = synth.hessian(K, 10)
    o = og.gptq(W, H)
    frame = oracle.quantize(W, "4o6")
    s_cols = np.repeat(scale_values(frame["scales"], frame["alpha"]), 16, axis=1)
    w = indep.as_f32(W).astype(np.float64)

    def weighted(codes):
        e = w - dequant(indep.unpack(codes), s_cols)
        return float(np.einsum("ij,jk,ik->", e, H, e))

    assert weighted(o["codes"]) < 0.8 * weighted(frame["codes"])


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        og.gptq(synth.normal_bf16(2, 32, 0), np.eye(16))


def test_calibration_second_moment_is_a_valid_input():
    """The generator's H: exactly symmetric, positive semi-definite (to rounding), dead inputs are whole
    zero rows and columns, and it is the scaled Gram matrix of its activations."""
    H = synth.hessian(80, 3, n=120, dead=3)
    assert np.array_equal(H, H.T)
    ev = np.linalg.eigvalsh(H)
    assert ev.min() > -1e-10 * ev.max()
    dead = np.flatnonzero(np.diag(H) == 0.0)
    assert dead.size == 3 and not H[dead].any() and not H[:, dead].any()
    X = synth.activations(120, 80, 3, dead=3)
    np.testing.assert_allclose(H, X.T @ X / 120, rtol=1e-12, atol=1e-12 * np.abs(H).max())
