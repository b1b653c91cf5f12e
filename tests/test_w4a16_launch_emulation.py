"""Host emulation of the W4A16 product's launches (CPU only, no device work).

For a set of shapes (the graph-capture cases, the eager parity cases and the benchmark's 4096 x 4096
cases) the launch plan comes from the library itself (nvfp4_matmul_plan, the function the launcher
calls). Every global and LDS address the three kernels form is then recomputed from the kernel source's
index arithmetic, over all work-groups, threads and K steps, and checked:
  * every load of X, codes and scales and every store of Y or of the split-K partials is inside its
    buffer; every LDS access is inside its array;
  * the XCD remap of work-group indices is a permutation;
  * the K slices partition [0, K) and every output (or partial of a slice) is written exactly once.
"""
import numpy as np
import pytest

import nvfp4_block_scaled_elem_amd as nv

BK = 64
LDS_STRIDE = BK + 8
GEMM_THREADS = 256


def tile_cfg(tm, tn):
    waves_n = 2 if tn == 128 else 1
    waves_m = 4 // waves_n
    wave_m, wave_n = tm // waves_m, tn // waves_n
    row_threads = GEMM_THREADS // tn
    return dict(waves_n=waves_n, wave_m=wave_m, wave_n=wave_n, mi=wave_m // 32, nj=wave_n // 32,
                row_threads=row_threads, thread_k=BK // row_threads)


def in_range(lo, hi, size, what):
    """Every byte range [lo, hi) lies in [0, size)."""
    lo, hi = np.asarray(lo), np.asarray(hi)
    assert lo.size == 0 or (lo.min() >= 0 and hi.max() <= size), f"{what}: [{lo.min()}, {hi.max()}) vs {size}"


def emulate_gemm(M, K, N, p):
    tm, tn, tiles_n, tiles, slices, kslice, grid = (p[k] for k in ("tm", "tn", "tiles_n", "tiles", "slices",
                                                                   "kslice", "grid"))
    c = tile_cfg(tm, tn)
    R, TK = c["row_threads"], c["thread_k"]
    assert grid == tiles * slices
    if slices == 1:
        assert kslice == K
    else:
        assert kslice % BK == 0 and slices * kslice >= K and (slices - 1) * kslice < K
    if slices > 1:
        assert p["part_bytes"] == slices * M * N * 4
    x_bytes, code_bytes, scale_bytes = M * K * 2, N * K // 2, N * K // 16
    out_elems = (slices * M * N) if slices > 1 else M * N
    written = np.zeros(out_elems, np.int32)
    tid = np.arange(GEMM_THREADS)
    wave, lane = tid >> 6, tid & 63
    remapped = []
    for blk in range(grid):
        b = (blk % 8) * (grid // 8) + blk // 8 if grid % 8 == 0 else blk
        remapped.append(b)
        sl, t = b // tiles, b % tiles
        m0, n0 = (t // tiles_n) * tm, (t % tiles_n) * tn
        kbeg, kend = sl * kslice, min(K, sl * kslice + kslice)
        assert kbeg < kend
        full = m0 + tm <= M and n0 + tn <= N and (kend - kbeg) % BK == 0
        k0 = np.arange(kbeg, kend, BK)[:, None]  # K steps x threads
        # X tile: TM / 32 loads of 8 bf16 per thread and step
        for q in range(tm // 32):
            idx = tid + q * GEMM_THREADS
            m, k = m0 + (idx >> 3), k0 + 8 * (idx & 7)
            ok = np.ones_like(k, bool) if full else (m < M) & (k < kend)
            e = (m * K + k)[ok]
            in_range(2 * e, 2 * e + 16, x_bytes, "X")
            if full:
                assert np.all(k + 8 <= K) and np.all(m < M)
            xl = (idx >> 3) * LDS_STRIDE + 8 * (idx & 7)
            in_range(xl, xl + 8, tm * LDS_STRIDE, "LDS xs")
        # weight tile: codes and scale bytes
        n, k = n0 + tid // R, k0 + TK * (tid % R)
        ok = np.ones_like(k, bool) if full else (n < N) & (k < kend)
        e = (n * K + k)
        if TK == 16:
            nb, ns = np.full_like(k, 8), np.full_like(k, 1)
        else:
            last16 = (~np.ones_like(k, bool)) if full else (k + 32 > kend)
            nb, ns = np.where(last16, 8, 16), np.where(last16, 1, 2)
        in_range((e // 2)[ok], (e // 2 + nb)[ok], code_bytes, "codes")
        in_range((e // 16)[ok], (e // 16 + ns)[ok], scale_bytes, "scales")
        assert np.all(e % 16 == 0)
        wl = (tid // R) * LDS_STRIDE + TK * (tid % R)
        in_range(wl, wl + TK, tn * LDS_STRIDE, "LDS ws")
        # MFMA operand reads
        wm, wn = (wave // c["waves_n"]) * c["wave_m"], (wave % c["waves_n"]) * c["wave_n"]
        for i in range(c["mi"]):
            assert np.all(wm + 32 * i + (lane & 31) < tm)
        for j in range(c["nj"]):
            assert np.all(wn + 32 * j + (lane & 31) < tn)
        assert 48 + 8 + 8 <= LDS_STRIDE  # kk + 8 * (lane / 32) + 8 <= BK
        # outputs
        mb, nbase = m0 + wm + 4 * (lane >> 5), n0 + wn + (lane & 31)
        for i in range(c["mi"]):
            for ee in range(16):
                r = 32 * i + 8 * (ee >> 2) + (ee & 3)
                for j in range(c["nj"]):
                    row, col = mb + r, nbase + 32 * j
                    ok = np.ones_like(row, bool) if full else (row < M) & (col < N)
                    assert np.all(row[ok] < M) and np.all(col[ok] < N)
                    idx = row[ok] * N + col[ok] + (sl * M * N if slices > 1 else 0)
                    in_range(idx, idx + 1, out_elems, "Y / partials")
                    np.add.at(written, idx, 1)
    assert sorted(remapped) == list(range(grid))
    assert np.all(written == 1), "an output is written twice or never"


def emulate_gemv(M, K, N, p):
    grid = p["grid"]
    chunks = -(-K // 2048)
    CH = 2 if chunks <= 2 else 4 if chunks <= 4 else 8
    threads, waves = 1024, 16
    assert grid == -(-N // waves)
    tid = np.arange(threads)
    lane, w = tid & 63, tid >> 6
    written = np.zeros(M * N, np.int32)
    for blk in range(grid):
        n = blk * waves + w
        for ch in range(CH):
            k = 32 * (lane + 64 * ch)
            ok = (n < N) & (k < K)
            e = n * K + k
            nb = np.where(k + 32 <= K, 16, 8)
            in_range((e // 2)[ok], (e // 2 + nb)[ok], N * K // 2, "codes")
            in_range((e // 16)[ok], (e // 16 + nb // 8)[ok], N * K // 16, "scales")
            valid = k < K
            nq = np.where(k + 32 <= K, 4, 2)
            for m in range(M):
                in_range((m * K + k)[valid], (m * K + k + 8 * nq)[valid], M * K, "LDS X")
        for m in range(M):
            rows = n[(lane == 63) & (n < N)]
            np.add.at(written, m * N + rows, 1)
    assert np.all(written == 1)


def emulate_skinny(M, K, N, p):
    grid, mt = p["grid"], p["tm"] // 16
    assert grid == -(-N // 16) and 16 * mt >= M > 16 * (mt - 1)
    threads, waves = 1024, 16
    tid = np.arange(threads)
    lane, w = tid & 63, tid >> 6
    r16, g = lane & 15, lane >> 4
    nch = -(-K // 128)
    written = np.zeros(M * N, np.int32)
    for blk in range(grid):
        n0 = blk * 16
        n = n0 + r16
        for c0 in range(0, nch, waves):
            c = c0 + w
            act = c < nch
            k = 128 * c + 32 * g
            ok = act & (n < N) & (k < K)
            e = n * K + k
            nb = np.where(k + 32 <= K, 16, 8)
            in_range((e // 2)[ok], (e // 2 + nb)[ok], N * K // 2, "codes")
            in_range((e // 16)[ok], (e // 16 + nb // 8)[ok], N * K // 16, "scales")
            for t in range(mt):
                m = 16 * t + r16
                for i in range(4):
                    okx = act & (m < M) & (k + 8 * i < K)
                    ex = (m * K + k + 8 * i)[okx]
                    in_range(2 * ex, 2 * ex + 16, M * K * 2, "X")
        for o in range(0, mt * 256):
            t, l, r = o >> 8, (o >> 2) & 63, o & 3
            nn, m = n0 + 4 * (l >> 4) + r, 16 * t + (l & 15)
            if nn < N and m < M:
                written[m * N + nn] += 1
    assert np.all(written == 1)


CAPTURED = [(1, 1024, 256), (1024, 1024, 256), (2100, 128, 256), (65536, 128, 256)]
EAGER_GEMM = [(65, 320, 40), (130, 528, 260), (128, 1024, 256), (300, 96, 136), (512, 160, 512), (260, 48, 1100),
              (513, 144, 200), (1024, 128, 256), (2048, 96, 130), (2049, 48, 136), (96, 1024, 256),
              (512, 1024, 256), (300, 128, 256)]
BENCH = [(256, 4096, 4096), (1024, 4096, 4096), (4096, 4096, 4096)]
SMALL = [(1, 1024, 256), (4, 16384, 40), (3, 6160, 9), (16, 4096, 64), (64, 2064, 100), (40, 48, 33),
         (4, 16400, 24), (48, 4112, 17)]


def run(M, K, N):
    p = nv.matmul_plan(M, K, N)
    assert p["part_bytes"] == nv.matmul_workspace_bytes(M, K, N)
    if p["kind"] == 0:
        emulate_gemv(M, K, N, p)
    elif p["kind"] == 1:
        emulate_skinny(M, K, N, p)
    else:
        emulate_gemm(M, K, N, p)
    return p


@pytest.mark.parametrize("M,K,N", CAPTURED)
def test_captured_shapes_stay_in_bounds(M, K, N):
    p = run(M, K, N)
    kinds = {(1, 1024, 256): (0, None), (1024, 1024, 256): (2, (128, 128, 4)), (2100, 128, 256): (2, (128, 128, 1)),
             (65536, 128, 256): (2, (256, 128, 1))}
    kind, tiles = kinds[(M, K, N)]
    assert p["kind"] == kind
    if tiles:
        assert (p["tm"], p["tn"], p["slices"]) == tiles


@pytest.mark.parametrize("M,K,N", EAGER_GEMM + BENCH)
def test_tiled_shapes_stay_in_bounds(M, K, N):
    assert run(M, K, N)["kind"] == 2


@pytest.mark.parametrize("M,K,N", SMALL)
def test_gemv_and_skinny_shapes_stay_in_bounds(M, K, N):
    assert run(M, K, N)["kind"] in (0, 1)


def test_workspace_query():
    assert nv.matmul_workspace_bytes(4096, 4096, 4096) == 0
    assert nv.matmul_workspace_bytes(1024, 1024, 256) == 4 * 1024 * 256 * 4
    assert nv.matmul_workspace_bytes(1024, 1000, 256) == 0  # K % 16 != 0 is rejected
