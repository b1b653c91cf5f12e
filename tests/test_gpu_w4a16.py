"""GPU W4A16 product with NVFP4 weights against the oracle (nvfp4_ref_matmul: exact products summed in
binary128). Identity and one-hot activations make every output a single exact product, so those cases
must match exactly; general activations are held to the fp32 accumulation bound
|y - y_exact| <= (K * 2^-23 + 2^-22) * alpha * sum_k |x * q * Delta| (+ 2^-8 |y| for bf16 output)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_elem_amd as nv
import oracle
import synth
from tests import indep

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def encoded_weights(n, k, seed, mode="4o6"):
    W = synth.normal_bf16(n, k, seed)
    codes, scales, alpha = nv.quantize(bf16_dev(W), mode, 2 if mode in ("cjso", "soar") else 0)
    torch.cuda.synchronize()
    return codes, scales, alpha


def check(X, codes, scales, alpha, out_dtype):
    M, K = X.shape
    N = codes.shape[0]
    say(f"w4a16 M={M} N={N} K={K} out={out_dtype}")
    Y = nv.matmul(bf16_dev(X), codes, scales, alpha, out_dtype=out_dtype)
    torch.cuda.synchronize()
    c, s, a = codes.cpu().numpy(), scales.cpu().numpy(), float(alpha.cpu()[0])
    ref = oracle.matmul(X, c, s, a, N)
    got = Y.float().cpu().numpy().astype(np.float64)
    x = indep.as_f32(X).astype(np.float64)
    wh = np.abs(oracle.dequantize(c, s, a, N, K))
    mag = np.abs(x) @ wh.T
    bound = (K * 2.0 ** -23 + 2.0 ** -22) * mag
    if out_dtype == torch.bfloat16:
        bound = bound + 2.0 ** -8 * np.abs(ref) + 1e-38
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"max excess {(err - bound).max()}"
    return got, ref


SHAPES = [(1, 256, 1024), (2, 96, 160), (3, 64, 272), (4, 130, 64),   # GEMV path (M <= 4), 2 chunks
          (1, 70, 4112), (3, 9, 6160), (2, 33, 12304), (4, 5, 8192),  # GEMV with 4 and 8 chunks of 2048 k
          (4, 37, 11008), (4, 40, 16384),  # X of 88 KB and 128 KB (the GEMV's LDS limit)
          (1, 21, 16400), (4, 24, 16400),  # past the GEMV's K limit: skinny MFMA path (M <= 64)
          (5, 200, 272), (7, 50, 9360), (9, 33, 7280), (12, 20, 1024), (13, 40, 5040), (16, 64, 4096),
          (16, 24, 4112), (17, 64, 512),
          (33, 50, 400), (48, 17, 4112), (64, 100, 2064), (20, 7, 16), (40, 33, 48),  # skinny: 1-4 tiles of 16 m
          (65, 40, 320), (130, 260, 528), (128, 256, 1024),  # 128 x 64 MFMA tiles (M <= 512), K split
          (300, 136, 96), (512, 512, 160), (260, 1100, 48),  # several 128 x 64 tiles (8 | tiles: remapped)
          (513, 200, 144), (1024, 256, 128), (2048, 130, 96),  # 128 x 128 tiles (M > 512 and fewer than
          (2049, 136, 48)]  # 512 tiles of 256 x 128; those are timed and sampled at 4096 x 4096 below)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_w4a16_matches_oracle(m, n, k, out_dtype):
    codes, scales, alpha = encoded_weights(n, k, seed=m + n + k)
    X = synth.normal_bf16(m, k, seed=3 * m + 1, std=1.0)
    check(X, codes, scales, alpha, out_dtype)


@pytest.mark.parametrize("k", [64, 160, 512])
@pytest.mark.parametrize("n", [32, 200])
def test_w4a16_identity_is_exact(n, k):
    """X = I (M = K > 4: the MFMA path) and its first rows (M <= 4: the GEMV path): one product per
    output, so the fp32 results equal the oracle's exactly."""
    codes, scales, alpha = encoded_weights(n, k, seed=n * k, mode="soar")
    eye = (np.eye(k, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for X in (eye, eye[:3] if k > 3 else eye):
        got, ref = check(X, codes, scales, alpha, torch.float32)
        assert np.array_equal(got, ref.astype(np.float32).astype(np.float64))


def test_w4a16_one_hot_rows_are_exact():
    n, k = 96, 256
    codes, scales, alpha = encoded_weights(n, k, seed=9)
    X = np.zeros((8, k), np.float32)
    for i in range(8):
        X[i, (37 * i + 5) % k] = (-1.0) ** i * (1.0 + i / 8.0)
    Xb = (X.view(np.uint32) >> 16).astype(np.uint16)
    for rows in (Xb[:2], Xb):
        got, ref = check(rows, codes, scales, alpha, torch.float32)
        assert np.array_equal(got, ref.astype(np.float32).astype(np.float64))


def test_w4a16_full_size_sample():
    """4096 x 4096 weights with M = 1 (GEMV), 8, 16 and 64 (skinny MFMA), 256 (128 x 64 tiles, K split),
    1024 (128 x 128 tiles) and 4096 (256 x 128 tiles, whole K): the bench's cases and the other tile
    shapes, sampled outputs against the oracle. Each output depends only on its own row of X, so every
    61st weight row is checked against every row of X (every 61st for M > 256)."""
    n = k = 4096
    W = synth.c2(0)
    codes, scales, alpha = nv.quantize(bf16_dev(W), "4o6")
    c, s, a = codes.cpu().numpy(), scales.cpu().numpy(), float(alpha.cpu()[0])
    rows = np.arange(0, n, 61)
    for m in (1, 8, 16, 64, 256, 1024, 4096):
        X = synth.normal_bf16(m, k, seed=m, std=1.0)
        say(f"w4a16 full size M={m}")
        Y = nv.matmul(bf16_dev(X), codes, scales, alpha, out_dtype=torch.float32)
        torch.cuda.synchronize()
        xrows = np.arange(0, m, 61) if m > 256 else np.arange(m)
        got = Y.cpu().numpy().astype(np.float64)[xrows][:, rows]
        X = np.ascontiguousarray(X[xrows])
        ref = oracle.matmul(X, c.reshape(n, k // 2)[rows], s.reshape(n, k // 16)[rows], a, rows.size)
        x = indep.as_f32(X).astype(np.float64)
        wh = np.abs(oracle.dequantize(c.reshape(n, k // 2)[rows], s.reshape(n, k // 16)[rows], a, rows.size, k))
        bound = (k * 2.0 ** -23 + 2.0 ** -22) * (np.abs(x) @ wh.T)
        assert np.all(np.abs(got - ref) <= bound)


def graph_replays_match_eager(cases, n=256):
    """Capture one product per case in one graph, replay it three times with eager work in between, and
    check that each replay equals the eager result."""
    w = {1024: encoded_weights(n, 1024, 21), 128: encoded_weights(n, 128, 23)}  # K = 128 never splits
    xs = {c: bf16_dev(synth.normal_bf16(c[0], c[1], seed=100 + c[0], std=1.0)) for c in cases}
    eager = {c: nv.matmul(xs[c], *w[c[1]]) for c in cases}
    torch.cuda.synchronize()
    outs = {c: torch.empty((c[0], n), dtype=torch.bfloat16, device="cuda") for c in cases}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in cases:
            nv.matmul(xs[c], *w[c[1]], out=outs[c])
    for rep in range(3):
        for y in outs.values():
            y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for c in cases:
            assert torch.equal(outs[c], eager[c]), (rep, c)
        nv.matmul(xs[cases[0]], *w[1024])  # eager work between replays
        torch.cuda.synchronize()


def test_w4a16_graph_replays_match_eager():
    """GEMV, skinny, 128 x 64 tiles with K split (stream-ordered scratch) and without, in one graph."""
    graph_replays_match_eager([(1, 1024), (16, 1024), (96, 1024), (512, 1024), (300, 128)])


@pytest.mark.skip(reason="this capture (128 x 128 tiles with and without K split, 256 x 128 tiles) ended "
                         "in a GPU memory fault once; the host emulation of every kernel address for these "
                         "shapes (tests/test_w4a16_launch_emulation.py) finds none out of bounds, and no "
                         "cause has been shown, so it stays off the GPU until one is")
def test_w4a16_graph_replays_match_eager_large_tiles():
    graph_replays_match_eager([(1, 1024), (1024, 1024), (2100, 128), (65536, 128)])


@pytest.mark.parametrize("M,K", [(1024, 1024), (2100, 128), (65536, 128)])
def test_w4a16_large_tiles_are_refused_under_capture(M, K):
    """The 128 x 128 and 256 x 128 tile forms return NVFP4_ERR_UNSUPPORTED on a capturing stream and
    enqueue nothing: no product runs here (these are the shapes of the skipped capture test, which also ran
    them eagerly before it faulted)."""
    n = 256
    plan = nv.matmul_plan(M, K, n)
    assert plan["kind"] == 2 and plan["tn"] == 128, plan
    codes, scales, alpha = encoded_weights(n, K, 31)
    X = bf16_dev(synth.normal_bf16(M, K, seed=5, std=1.0))
    out = torch.empty((M, n), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, nv.matmul_workspace_bytes(M, K, n)), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        with pytest.raises(nv.NVFP4Error, match=r"\(-6\)"):
            nv.matmul(X, codes, scales, alpha, out=out, workspace=ws)
    del g
    torch.cuda.synchronize()


def test_w4a16_on_a_side_stream():
    n, k = 200, 512
    codes, scales, alpha = encoded_weights(n, k, 22)
    X = bf16_dev(synth.normal_bf16(40, k, seed=7, std=1.0))
    ref = nv.matmul(X, codes, scales, alpha)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        Y = nv.matmul(X, codes, scales, alpha)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(Y, ref)
