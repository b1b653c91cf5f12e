"""Seeded synthetic weight matrices for the tests and the benchmark.

This module only draws inputs. It holds none of the quantizer's arithmetic and is the one piece of code
that the oracle's tests and the GPU path's tests share. Everything is generated on the host with numpy's
PCG64 generator keyed by (seed, matrix id, stream), so a given call returns the same bytes on every
machine with this numpy.

bf16 matrices are returned as ``uint16`` arrays of bf16 bit patterns (binary64 draw -> binary32 ->
bf16, each step round-to-nearest-even); fp32 matrices as ``float32``.

Workloads (weights of real models are not available; these stand in for them):
  * ``c1``: 256 x 1024 fp32, i.i.d. N(0, 0.02^2).
  * ``c2``: 4096 x 4096 bf16 attention-projection shape: Student-t (nu = 4) scaled to std 0.02, with
    round(0.001 * cols) whole columns multiplied by 20 (about 0.1 % of the entries) as outlier columns.
  * ``c3``: 14336 x 4096 and 4096 x 14336 bf16 MLP up/down shapes: N(0, 0.015^2) with each row's std
    multiplied by 2^U(-1, 1), i.e. log-uniform on [0.5, 2].
  * ``c5``: one linear layer of a 7B-shaped transformer (q, k, v, o 4096 x 4096; gate, up 11008 x 4096;
    down 4096 x 11008) bf16, Student-t (nu = 5) scaled to std 0.02, seeded by the layer index.
  * ``soar_tie_matrix``: fp32 blocks constructed so that the decoupled search ends in an exact tie
    between its two reconstruct scales (described at the function).
  * ``activations`` / ``hessian``: calibration inputs of a linear layer for GPTQ (no real activations
    are available): per-feature scales 2^U(-2, 2), a rank-8 component shared by all features so that
    they correlate, optionally some features that are always zero; ``hessian`` returns their second
    moment X^T X / n in binary64, the matrix GPTQ takes as input.
"""
from __future__ import annotations

import numpy as np

C5_SHAPES = {
    "q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
    "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008),
}
C5_ORDER = ("q", "k", "v", "o", "gate", "up", "down")


def rng(seed: int, matrix_id: int = 0, stream: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(matrix_id), int(stream)])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite binary32 values to bf16 (nearest, ties to even) and return the bit patterns."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def student_t(g: np.random.Generator, nu: float, shape, std: float) -> np.ndarray:
    """Student-t draws scaled so that the population std is ``std`` (requires nu > 2)."""
    return g.standard_t(nu, size=shape) * (std / np.sqrt(nu / (nu - 2.0)))


def c1(seed: int = 0) -> np.ndarray:
    g = rng(seed, 0)
    return (g.standard_normal((256, 1024)) * 0.02).astype(np.float32)


def c2(seed: int = 0, rows: int = 4096, cols: int = 4096) -> np.ndarray:
    g = rng(seed, 0)
    w = student_t(g, 4.0, (rows, cols), 0.02)
    k = int(round(0.001 * cols))
    cols_out = rng(seed, 0, 1).permutation(cols)[:k]
    w[:, cols_out] *= 20.0
    return bf16_bits(w.astype(np.float32))


def c3(which: int, seed: int = 0, rows: int = 0) -> np.ndarray:
    """`rows` > 0: only the first rows of the matrix (the same values; the draws are made in row order)."""
    full, cols = ((14336, 4096), (4096, 14336))[which]
    rows = rows or full
    g = rng(seed, which)
    sigma = 0.015 * np.exp2(rng(seed, which, 1).uniform(-1.0, 1.0, size=(rows, 1)))
    return bf16_bits((g.standard_normal((rows, cols)) * sigma).astype(np.float32))


def c5(layer: int, name: str, rows: int = 0) -> np.ndarray:
    """`rows` > 0: only the first rows of the matrix (the same values; the draws are made in row order)."""
    full, cols = C5_SHAPES[name]
    rows = rows or full
    g = rng(layer, C5_ORDER.index(name))
    return bf16_bits(student_t(g, 5.0, (rows, cols), 0.02).astype(np.float32))


def normal_bf16(rows: int, cols: int, seed: int, std: float = 0.02) -> np.ndarray:
    return bf16_bits((rng(seed, 7).standard_normal((rows, cols)) * std).astype(np.float32))


def normal_f32(rows: int, cols: int, seed: int, std: float = 0.02) -> np.ndarray:
    return (rng(seed, 8).standard_normal((rows, cols)) * std).astype(np.float32)


# Two blocks in units of alpha = 2^-12, eta = 2^-18 (every value is a binary32 number). Under the max rule
# (no CJSO rounds) block A gets Delta_c = 15 with the reconstruct pair {15, 16}, block B Delta_c = 15 with
# {14, 15}. The element 52.5 - eta lies just below the E2M1 midpoint 3.5 at scale 15; binary32 rounding of
# its scaled value lands on 3.5, so the incumbent codes it 4 where 3 is nearer, and candidates with
# Delta_q slightly above 15 beat the incumbent. The other elements are chosen so that the least error at
# either reconstruct scale is exactly the same number: the eta terms cancel (the 3 eta and -11 eta
# elements) and the remaining squares balance (the 30 and 15s in A, the 60 and 45 in B).
_ETA = 2.0 ** -18
SOAR_TIE_BLOCKS = {
    "A": [91.0, 52.5 - _ETA, 17.0 + 3 * _ETA, 30.0] + [15.0] * 11 + [0.0],
    "B": [89.0, 52.5 - _ETA, 12.0 - 11 * _ETA, 60.0, 45.0] + [0.0] * 11,
}
SOAR_TIE_ALPHA = 2.0 ** -12


def soar_tie_matrix(seed: int = 0, rows: int = 8, cols: int = 256):
    """fp32 [rows, cols] whose global max is 6 * 448 * 2^-12 (so the max rule's alpha is exactly 2^-12),
    holding copies of SOAR_TIE_BLOCKS (elements permuted, signs drawn per element) between N(0, 0.02^2)
    blocks. Returns (W, kinds) with kinds[b] = "A", "B" or "" for block b in row-major block order."""
    g = rng(seed, 10)
    nb = rows * cols // 16
    kinds = g.choice(np.array(["A", "B", ""]), size=nb, p=[0.4, 0.4, 0.2])
    kinds[0] = ""
    W = (g.standard_normal((nb, 16)) * 0.02).astype(np.float32)
    for b in range(nb):
        if kinds[b]:
            v = np.array(SOAR_TIE_BLOCKS[kinds[b]], np.float64)[g.permutation(16)]
            W[b] = (v * g.choice([-1.0, 1.0], size=16) * SOAR_TIE_ALPHA).astype(np.float32)
    W[0, int(g.integers(16))] = np.float32(6 * 448 * SOAR_TIE_ALPHA) * np.float32(g.choice([-1.0, 1.0]))
    return W.reshape(rows, cols), [str(k) for k in kinds]


def activations(n: int, cols: int, seed: int, dead: int = 0) -> np.ndarray:
    """n calibration input vectors of a layer with `cols` inputs, binary64 [n, cols]."""
    g = rng(seed, 9)
    sigma = np.exp2(g.uniform(-2.0, 2.0, size=cols))
    shared = g.standard_normal((n, 8)) @ g.standard_normal((8, cols)) / np.sqrt(8.0)
    X = (g.standard_normal((n, cols)) + 0.5 * shared) * sigma
    if dead:
        X[:, rng(seed, 9, 1).permutation(cols)[:dead]] = 0.0
    return X


def hessian(cols: int, seed: int, n: int = 0, dead: int = 0) -> np.ndarray:
    """X^T X / n of `activations` (n = 2 cols unless given): symmetric positive semi-definite, binary64."""
    n = n or 2 * cols
    X = activations(n, cols, seed, dead)
    H = X.T @ X / n
    return (H + H.T) / 2.0  # exactly symmetric whatever order the product summed in
