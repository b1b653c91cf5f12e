"""Independent checks used to pin the oracle: brute-force searches and library routines written apart
from it, so that a slip in the oracle's own code shows up as a disagreement."""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_e2m1() -> np.ndarray:
    vals = []
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, v = line.split()
                vals.append((int(code), float(v)))
    vals.sort()
    return np.array([v for _, v in vals], np.float64)


def golden_constants() -> dict:
    out = {}
    with open(os.path.join(GOLDEN, "constants.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                name, v = line.split()[:2]
                out[name] = float(v)
    return out


E2M1_VALUES = golden_e2m1()
GRID = E2M1_VALUES[:8]


def brute_e2m1(x: np.ndarray) -> np.ndarray:
    """Nearest of the eight magnitudes by exhaustive comparison, ties to the even code, sign in bit 3
    for nonzero negative results, NaN -> 0, infinities -> 6."""
    x = np.asarray(x, np.float32).reshape(-1)
    with np.errstate(invalid="ignore"):
        t = np.abs(x.astype(np.float64))
    # beyond 16 the nearest magnitude is 6 whatever t is; clamping keeps the distances below exact
    t = np.where(t > 16.0, 16.0, t)
    d = np.abs(t[:, None] - GRID[None, :])  # exact: t has 24 bits, grid values 3
    best = d.min(axis=1)
    cand = d == best[:, None]
    idx = cand.argmax(axis=1)
    two = cand.sum(axis=1) == 2
    idx = np.where(two & (idx % 2 == 1), idx + 1, idx)
    idx = np.where(np.isnan(t), 0, idx)
    neg = np.signbit(x) & (idx > 0)
    return (idx | np.where(neg, 8, 0)).astype(np.uint8)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return E2M1_VALUES[np.asarray(codes, np.int64) & 15]


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 byte -> value through torch's float8_e4m3fn."""
    c = torch.from_numpy(np.ascontiguousarray(np.asarray(codes, np.uint8)))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0..126


def brute_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest of the 127 non-negative finite E4M3 values by exhaustive comparison, ties to the even
    code (saturates at 448 because nothing larger is finite)."""
    v = np.asarray(v, np.float64).reshape(-1)
    out = np.empty(v.size, np.uint8)
    for s in range(0, v.size, 1 << 16):
        vv = v[s:s + (1 << 16)]
        d = np.abs(vv[:, None] - E4M3_POS[None, :])
        best = d.min(axis=1)
        cand = d == best[:, None]
        idx = cand.argmax(axis=1)
        two = cand.sum(axis=1) == 2
        idx = np.where(two & (idx % 2 == 1), idx + 1, idx)
        out[s:s + (1 << 16)] = idx
    return out


def torch_e4m3(v_f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v_f32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def nearest_f32(fr: Fraction) -> np.float32:
    """The binary32 value nearest to a rational (ties to even), by exact comparison of neighbours."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        if best is None or d < best[0] or (d == best[0] and (int(np.float32(cand).view(np.uint32)) & 1) == 0):
            best = (d, cand)
    return np.float32(best[1])


def quantize_block_np(w16: np.ndarray, alpha: float, delta: float) -> np.ndarray:
    """Binary32 scaled value x = w * (1/(alpha*delta)) followed by the brute-force E2M1 search."""
    w16 = np.asarray(w16, np.float32)
    s = np.float32(alpha) * np.float32(delta)
    if s == 0:
        return np.zeros(w16.shape, np.uint8)
    r = np.float32(1.0) / s
    return brute_e2m1((w16 * r).astype(np.float32)).reshape(w16.shape)


def block_err_np(w16: np.ndarray, codes16: np.ndarray, alpha: float, delta_d: float) -> float:
    q = e2m1_decode(codes16)
    d = np.asarray(w16, np.float64) - q * float(alpha) * float(delta_d)
    return float(np.sum(d * d))


def unpack(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, np.uint8)
    return np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


def as_f32(W: np.ndarray) -> np.ndarray:
    if W.dtype == np.uint16:
        return (W.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(W, np.float32)


def block_errors(W: np.ndarray, codes: np.ndarray, scales: np.ndarray, alpha: float) -> np.ndarray:
    """Per-block squared error in binary64 from an output triple (independent of the oracle)."""
    w = as_f32(W).astype(np.float64).reshape(-1, 16)
    q = e2m1_decode(unpack(codes)).reshape(-1, 16)
    d = e4m3_decode(np.asarray(scales).reshape(-1))[:, None]
    e = w - q * float(alpha) * d
    return np.sum(e * e, axis=1)


def on_grid_matrix(rows: int, cols: int, alpha_exp: int, seed: int, dtype=np.uint16):
    """W = alpha0 * Delta_i * Q_ij exactly, alpha0 = 2^alpha_exp, with Delta_i random E4M3 values, Q
    random E2M1 values, a +-6 in every block and block 0 at Delta = 448 (so max|W| = 6*448*alpha0).
    Returns (W, alpha0, scale codes [rows, cols//16], codes [rows, cols])."""
    g = np.random.default_rng(seed)
    nb = cols // 16
    dcode = g.integers(8, 120, size=(rows, nb)).astype(np.uint8)
    dcode[0, 0] = 0x7E
    q = g.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    q[q == 8] = 0  # negative zero is never produced
    pos = g.integers(0, 16, size=(rows, nb))
    sign = g.integers(0, 2, size=(rows, nb)).astype(np.uint8) * 8
    qb = q.reshape(rows, nb, 16)
    np.put_along_axis(qb, pos[..., None], (7 | sign)[..., None], axis=2)
    q = qb.reshape(rows, cols)
    alpha0 = 2.0 ** alpha_exp
    w = e2m1_decode(q) * np.repeat(e4m3_decode(dcode), 16, axis=1) * alpha0
    w32 = w.astype(np.float32)
    assert np.all(w32.astype(np.float64) == w)
    if dtype == np.uint16:
        bits = (w32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        assert np.all((bits.astype(np.uint32) << np.uint32(16)) == w32.view(np.uint32))
        return bits, alpha0, dcode, q
    return w32, alpha0, dcode, q
