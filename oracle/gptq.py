"""GPTQ with the FourOverSix block scales fixed first: the CPU oracle.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this module. The product package never imports it.

Sources:
* FourOverSix page, section "03 our integration": each block's scale is estimated, its M = 6 / M = 4
  reconstruction errors are compared and the better scale is chosen; only then do the GPTQ weight
  iterations run, inside that fixed frame, so scale choice and GPTQ do not interact.
* GPTQ (Frantar, Ashkboos, Hoefler, Alistarh, 2022), the algorithm the page names: given the second
  moment H of a layer's inputs, inputs whose diagonal entry is zero are dead (their weights are set to
  zero and the diagonal entry to one), H is damped by a fraction of its mean diagonal, U is the upper
  Cholesky factor of H^-1, and the columns are quantised in order, each column's error divided by
  U_jj and spread over the later columns along row j of U.

Readings (the pages leave these open):
* The frozen frame is the whole FourOverSix result on the original W: the per-block E4M3 scales and
  the global alpha. GPTQ chooses the codes only.
* Arithmetic is binary64 throughout. A column is quantised as in the format: s = fl32(alpha * Delta)
  (binary32, as every mode computes it), x = w / s in binary64, the E2M1 magnitude by the nearest-value
  thresholds (ties to the even code), sign in bit 3; s = 0 gives code 0. The dequantised value is
  G[code] * s (exact in binary64).
* Columns in their natural order (no activation reordering); the unblocked update (GPTQ's lazy
  batches only regroup the same sums).
"""
from __future__ import annotations

import numpy as np

from . import lib, quantize

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_index(a: np.ndarray) -> np.ndarray:
    """Index of the nearest E2M1 magnitude to a >= 0 (ties to the even index; 6 beyond)."""
    return ((a > 0.25).astype(np.int64) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5)
            + (a > 5.0))


def block_scale_values(scales: np.ndarray, alpha: float) -> np.ndarray:
    """s = fl32(alpha * Delta) per block, as binary64 values."""
    e4m3 = np.array([lib().nvfp4_ref_e4m3_value(c) for c in range(256)], np.float64)
    delta = e4m3[np.asarray(scales, np.uint8)].astype(np.float32)  # E4M3 values are binary32 numbers
    return (np.float32(alpha) * delta).astype(np.float64)


def damped_hessian(H: np.ndarray, percdamp: float):
    """GPTQ's preparation of H: dead inputs (zero diagonal) get diagonal 1, then every diagonal entry
    gains percdamp * mean(diag). Returns (the damped copy, the dead mask)."""
    H = np.array(H, np.float64, copy=True)
    K = H.shape[0]
    dead = np.diag(H) == 0.0
    H[dead, dead] = 1.0
    H[np.arange(K), np.arange(K)] += percdamp * np.mean(np.diag(H))
    return H, dead


def inverse_cholesky_upper(Hd: np.ndarray) -> np.ndarray:
    """U upper triangular with U^T U = Hd^-1: H^-1 from the Cholesky factor of H, then its own upper
    Cholesky factor."""
    L = np.linalg.cholesky(Hd)
    Linv = np.linalg.inv(L)
    Hinv = Linv.T @ Linv
    return np.linalg.cholesky(Hinv).T


def gptq(W: np.ndarray, H: np.ndarray, percdamp: float = 0.01, rows=None, *, trace: bool = False):
    """GPTQ codes for W ([R, K] bf16 bits as uint16, or float32) under the frozen FourOverSix frame.

    H is the [K, K] input second moment (binary64). `rows` limits the column sweep to those rows (each
    row's sweep depends only on its own weights, its block scales and U). Returns a dict with codes
    ([len(rows), K/2], low nibble even column), scales and alpha (the FourOverSix ones, all rows) and,
    with trace, the value each column was quantised from (`target`, binary64 [len(rows), K])."""
    W = np.ascontiguousarray(W)
    R, K = W.shape
    H = np.asarray(H, np.float64)
    if H.shape != (K, K) or K % 16:
        raise ValueError("H must be [K, K] for W [R, K] with K % 16 == 0")
    frame = quantize(W, "4o6")  # block scales and alpha first
    scales, alpha = frame["scales"], frame["alpha"]
    Hd, dead = damped_hessian(H, percdamp)
    U = inverse_cholesky_upper(Hd)

    sel = np.arange(R) if rows is None else np.asarray(rows, np.int64)
    Wf = (W.astype(np.uint32) << 16).view(np.float32) if W.dtype == np.uint16 else W
    w = Wf[sel].astype(np.float64)
    w[:, dead] = 0.0
    s = block_scale_values(scales[sel], alpha)
    code = np.zeros((sel.size, K), np.uint8)
    target = np.zeros((sel.size, K)) if trace else None
    for j in range(K):
        sj = s[:, j // 16]
        t = w[:, j]
        if trace:
            target[:, j] = t
        live = sj > 0.0
        x = np.where(live, t / np.where(live, sj, 1.0), 0.0)
        idx = np.where(live, _e2m1_index(np.abs(x)), 0)
        neg = (x < 0.0) & (idx > 0)
        code[:, j] = (idx | np.where(neg, 8, 0)).astype(np.uint8)
        deq = np.where(neg, -1.0, 1.0) * E2M1_MAGNITUDES[idx] * sj
        d = (t - deq) / U[j, j]
        w[:, j + 1:] -= np.outer(d, U[j, j + 1:])
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    out = {"codes": packed, "scales": scales, "alpha": alpha}
    if trace:
        out["target"] = target
    return out
