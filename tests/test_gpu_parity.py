"""GPU parity: the HIP path (through the C ABI) against the oracle, element by element.

Small and ragged shapes are compared with the oracle run live. Full-size workloads (4096 x 4096,
14336 x 4096, 4096 x 14336 and three matrices of a 7B-shaped layer) are compared with digests and
sampled blocks that tests/golden/make_golden.py wrote from the oracle. Modes MAX and FourOverSix must be
bit-exact (codes, scales, alpha, M=4 choices); CJSO and SOAR are held to the same bar here, which is
stricter than the stated tolerance (alpha within 1e-6 relative, codes and scales on at least 99.99 % of
blocks, MSE within 1e-5 relative) — the tolerance checks run first so a failure says which bar broke.
"""
import functools
import hashlib
import json
import os
import sys

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_elem_amd as nv
import oracle
import synth
from tests import indep

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    nv.lib()
    return torch.device("cuda:0")


def to_dev(W: np.ndarray) -> torch.Tensor:
    if W.dtype == np.uint16:
        return torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(W).cuda()


def run(W: np.ndarray, mode: str, iters: int = 0, dev_W=None, full_search=False, init="max", grid=None,
        dd_rule="cjso"):
    say(f"gpu quantize mode={mode} iters={iters} shape={W.shape} dtype={W.dtype} full_search={full_search} "
        f"init={init} grid={grid} dd_rule={dd_rule}")
    Wd = to_dev(W) if dev_W is None else dev_W
    rows, cols = W.shape
    mch = torch.zeros((rows, cols // 16), dtype=torch.uint8, device="cuda") if mode == "4o6" else None
    stats = torch.zeros(4, dtype=torch.int32, device="cuda")
    codes, scales, alpha = nv.quantize(Wd, mode, iters, mchoice=mch, stats=stats, full_search=full_search,
                                       init=init, grid=grid, dd_rule=dd_rule)
    torch.cuda.synchronize()
    out = {"codes": codes.cpu().numpy(), "scales": scales.cpu().numpy(), "alpha": float(alpha.cpu()[0]),
           "stats": stats.cpu().numpy()}
    if mch is not None:
        out["mchoice"] = mch.cpu().numpy()
    return out


def f32_bits(x):
    return int(np.float32(x).view(np.uint32))


def assert_tolerance(W, g, r):
    """The stated CJSO/SOAR bar, checked before bit-exactness so a failure names the broken bar."""
    if np.isnan(r["alpha"]):
        assert np.isnan(g["alpha"])
        return
    assert abs(g["alpha"] - r["alpha"]) <= 1e-6 * abs(r["alpha"])
    same = np.all(g["codes"].reshape(-1, 8) == r["codes"].reshape(-1, 8), axis=1) & \
        (g["scales"].reshape(-1) == r["scales"].reshape(-1))
    assert same.mean() >= 0.9999, f"{(~same).sum()} blocks differ"
    mg = oracle.mse(W, g["codes"], g["scales"], g["alpha"])
    mr = oracle.mse(W, r["codes"], r["scales"], r["alpha"])
    assert abs(mg - mr) <= 1e-5 * max(mr, 1e-300)


def assert_exact(g, r, mode):
    assert f32_bits(g["alpha"]) == f32_bits(r["alpha"]) or (np.isnan(g["alpha"]) and np.isnan(r["alpha"]))
    bad = np.nonzero(np.any(g["codes"].reshape(-1, 8) != r["codes"].reshape(-1, 8), axis=1) |
                     (g["scales"].reshape(-1) != r["scales"].reshape(-1)))[0]
    assert bad.size == 0, f"{mode}: {bad.size} blocks differ, first {bad[:8]}"
    if mode == "4o6":
        assert np.array_equal(g["mchoice"], r["mchoice"])
        assert int(g["stats"][1]) == int(r["mchoice"].sum())


def compare_live(W, mode, iters=0):
    g = run(W, mode, iters)
    r = oracle.quantize(W, mode, iters)
    if mode in ("cjso", "soar"):
        assert_tolerance(W, g, r)
    assert_exact(g, r, mode)
    return g, r


# ----------------------------------------------------------------------- live oracle, small sizes

@pytest.mark.parametrize("mode,iters", [("max", 0), ("4o6", 0), ("cjso", 8), ("soar", 8)])
def test_c1_fp32(mode, iters):
    compare_live(synth.c1(0), mode, iters)


RAGGED = [(1, 16), (3, 48), (37, 272), (130, 1040), (257, 4112)]


@pytest.mark.parametrize("shape", RAGGED)
@pytest.mark.parametrize("mode,iters", [("max", 0), ("4o6", 0), ("cjso", 0), ("cjso", 3), ("soar", 0), ("soar", 2)])
def test_ragged_bf16(shape, mode, iters):
    W = synth.bf16_bits(synth.student_t(synth.rng(sum(shape), 3), 4.0, shape, 0.02).astype(np.float32))
    compare_live(W, mode, iters)


@pytest.mark.parametrize("mode", ["max", "4o6", "cjso", "soar"])
def test_ragged_fp32(mode):
    compare_live(synth.normal_f32(53, 336, seed=4), mode, 3)


@pytest.mark.parametrize("dtype", [np.uint16, np.float32])
@pytest.mark.parametrize("mode", ["max", "4o6", "cjso", "soar"])
def test_on_grid_round_trip(dtype, mode):
    W, alpha0, dcode, q = indep.on_grid_matrix(16, 512, -9, seed=21, dtype=dtype)
    g = run(W, mode, 3)
    assert g["alpha"] == alpha0
    assert np.array_equal(g["scales"], dcode)
    assert np.array_equal(indep.unpack(g["codes"]), q)


def test_4o6_constructed_choices():
    alpha0 = 2.0 ** -10
    b0 = np.zeros(16); b0[0] = 6 * 448 * alpha0; b0[1:4] = np.array([1, 2, 3]) * alpha0
    b1 = np.array([4, 3, 1.5, 1, 0.5, 2, 0, -4, -3, -1.5, 1, 0.5, 2, 3, 4, 0]) * 3 * alpha0
    b2 = np.array([6, 0.5, 1, 1.5, 0.5, -0.5, 2, 3, 0.5, 1, 1.5, -6, 0.5, 1, 0, 0.5]) * 5 * alpha0
    b3 = np.array([6, 5, 1, 2, 0, 3.3, 1, 1, 2, 2, 1, 0, 0, 0, 0, 1]) * 448 * alpha0
    W = np.concatenate([b0, b1, b2, b3]).reshape(1, 64).astype(np.float32)
    g, _ = compare_live(W, "4o6")
    assert list(g["mchoice"].reshape(-1)) == [0, 1, 0, 0]


# ---------------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("mode", ["max", "4o6", "cjso", "soar"])
@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite(mode, bad):
    W = synth.normal_f32(8, 64, seed=1)
    W[5, 33] = bad
    g = run(W, mode, 2)
    assert np.isnan(g["alpha"]) and not g["codes"].any() and not g["scales"].any()
    assert g["stats"][0] & nv.STATUS_NONFINITE
    Wb = synth.bf16_bits(synth.normal_f32(8, 64, seed=1))
    Wb[2, 7] = {np.nan: 0x7FC0, np.inf: 0x7F80, -np.inf: 0xFF80}[bad] if not np.isnan(bad) else 0x7FC0
    g = run(Wb, mode, 2)
    assert np.isnan(g["alpha"]) and not g["codes"].any() and not g["scales"].any()


@pytest.mark.parametrize("mode", ["max", "4o6", "cjso", "soar"])
def test_zero_and_tiny(mode):
    W = np.zeros((4, 64), np.uint16)
    W[1, 3] = 0x8000
    g = run(W, mode, 2)
    assert g["alpha"] == 0.0 and not g["codes"].any() and not g["scales"].any() and g["stats"][0] == 0
    W = synth.normal_f32(4, 64, seed=2)
    W[1, 16:32] = 0.0
    W[2, 32:48] *= 1e-6
    compare_live(W, mode, 2)
    compare_live((synth.normal_f32(2, 32, seed=3) * 1e-36).astype(np.float32), mode, 1)
    compare_live((synth.normal_f32(2, 32, seed=4) * 1e30).astype(np.float32), mode, 1)
    big = synth.normal_bf16(2, 32, seed=5, std=1e30)
    compare_live(big, mode, 1)


@pytest.mark.parametrize("mode,iters", [("max", 0), ("4o6", 0), ("cjso", 3), ("soar", 0), ("soar", 3)])
def test_every_output_byte_written(mode, iters):
    """Outputs start as a pattern no quantiser writes (0xA5), so a block the kernels skip shows. The matrix
    has whole zero blocks (scale 0, whose codes the search leaves to nobody else), a zero row and
    ordinary blocks, over enough blocks for several loop iterations per thread."""
    W = synth.normal_bf16(96, 4096, 31)
    W[5, :] = 0
    W[7, 16:48] = 0
    W[9, 4080:] = 0
    W[40:42, ::7] = 0
    Wd = to_dev(W)
    rows, cols = W.shape
    codes = torch.full((rows, cols // 2), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, cols // 16), 0xA5, dtype=torch.uint8, device="cuda")
    alpha = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    mch = torch.full((rows, cols // 16), 0xA5, dtype=torch.uint8, device="cuda") if mode == "4o6" else None
    stats = torch.zeros(4, dtype=torch.int32, device="cuda")
    say(f"gpu quantize (outputs pre-filled) mode={mode} iters={iters} shape={W.shape}")
    nv.quantize(Wd, mode, iters, codes=codes, scales=scales, alpha=alpha, mchoice=mch, stats=stats)
    torch.cuda.synchronize()
    g = {"codes": codes.cpu().numpy(), "scales": scales.cpu().numpy(), "alpha": float(alpha.cpu()[0]),
         "stats": stats.cpu().numpy()}
    if mch is not None:
        g["mchoice"] = mch.cpu().numpy()
    r = oracle.quantize(W, mode, iters)
    assert (g["scales"][5] == 0).all() and (g["codes"][5] == 0).all()
    assert_exact(g, r, mode)


def edge_rows_bf16(seed: int) -> np.ndarray:
    """16 x 4096 bf16 rows of the blocks the quantisers treat apart: ordinary Student-t blocks, a row scaled
    down until its scales fall below E4M3's normal range, whole zero blocks and a zero row, blocks with one
    large element among small ones (their least-squares scale is far below max|w| / 6, so the binary32 sums
    leave their exactness window), outliers, and rows at other magnitudes."""
    x = synth.student_t(synth.rng(seed, 7), 4.0, (16, 4096), 0.02).astype(np.float32)
    x[1] *= 1e-2  # scales in E4M3's subnormal range
    x[2, 256:512] = 0.0
    blk = x[3].reshape(-1, 16)
    blk[::2, 1:] *= 1e-3
    x[4, ::97] *= 300.0
    x[5] = 0.0
    x[6] *= 3e-3
    x[7, ::5] = 0.0
    x[8] *= 1e-6  # scales that round to zero
    return synth.bf16_bits(x)


@pytest.mark.parametrize("case", ["mixed", "tiny"])
@pytest.mark.parametrize("mode,iters", [("max", 0), ("4o6", 0), ("cjso", 3), ("soar", 3)])
def test_tiled_edge_blocks_two_per_thread(case, mode, iters):
    """The edge blocks at a size where every pass gives each thread two or more blocks, so the paired
    common path and its per-block fallbacks run: the 16 x 4096 rows above, tiled 128 times by rows (2048 x
    4096). Tiling by whole rows leaves alpha unchanged in every mode (the global max is the same; the CJSO
    sums all scale by the tile count, so their quotient does not move), and each block's outputs depend
    only on the block and alpha, so the result must be the oracle's result for the small matrix, tiled.
    "tiny" scales everything by 1e-36, so alpha is subnormal and the scales' reciprocals overflow."""
    small = edge_rows_bf16(11)
    if case == "tiny":
        small = synth.bf16_bits(synth.bf16_to_f32(small) * np.float32(1e-36))
    r = oracle.quantize(small, mode, iters)
    big = np.tile(small, (128, 1))
    g = run(big, mode, iters)
    assert f32_bits(g["alpha"]) == f32_bits(r["alpha"])
    for key in ("codes", "scales") + (("mchoice",) if mode == "4o6" else ()):
        want = np.tile(r[key], (128, 1))
        bad = np.flatnonzero(np.any((g[key] != want).reshape(g[key].shape[0], -1), axis=1))
        assert bad.size == 0, f"{key}: rows {bad[:8]} differ"


@pytest.mark.parametrize("case", ["mixed", "tiny"])
@pytest.mark.parametrize("variant", ["full_scan", "grid", "quant", "lsq"])
def test_tiled_edge_blocks_search_variants(case, variant):
    """The same tiled edge rows through the search's other forms: the full scan (against the page's search
    in the oracle), another grid, and the two variant reconstruct-pair rules (against the oracle's
    configurable search). Each form has its own instantiation with its own prologue."""
    small = edge_rows_bf16(11)
    if case == "tiny":
        small = synth.bf16_bits(synth.bf16_to_f32(small) * np.float32(1e-36))
    kw = {"full_scan": dict(full_search=True), "grid": dict(grid=(100, 200, 201)),
          "quant": dict(dd_rule="quant"), "lsq": dict(dd_rule="lsq")}[variant]
    if variant == "full_scan":
        r = oracle.quantize(small, "soar", 3)
    else:
        r = oracle.quantize_search(small, 3, grid=kw.get("grid", oracle.PAGES_GRID),
                                   dd_rule=kw.get("dd_rule", "cjso"))
    big = np.tile(small, (128, 1))
    g = run(big, "soar", 3, **kw)
    assert f32_bits(g["alpha"]) == f32_bits(r["alpha"])
    for key in ("codes", "scales"):
        want = np.tile(r[key], (128, 1))
        bad = np.flatnonzero(np.any((g[key] != want).reshape(g[key].shape[0], -1), axis=1))
        assert bad.size == 0, f"{key}: rows {bad[:8]} differ"


def test_saturating_and_subnormal_scales():
    # blocks whose max-rule scale lands on 320..416 (FourOverSix M=4 scale saturates) and blocks whose
    # scales are E4M3 subnormals
    g = np.random.default_rng(8)
    rows = []
    top = np.zeros(16); top[0] = 1.0
    rows.append(top)
    for d in (320, 352, 384, 416, 300, 2 ** -7, 2 ** -8, 3 * 2 ** -9, 2 ** -9):
        b = g.uniform(-1, 1, 16) * d / 448.0
        b[0] = d / 448.0
        rows.append(b)
    W = np.concatenate(rows).reshape(1, -1).astype(np.float32)
    for mode in ("max", "4o6", "cjso", "soar"):
        compare_live(W, mode, 2)


# -------------------------------------------------------------------------------- determinism

def test_determinism_and_streams():
    W = synth.c2(0, rows=512, cols=2048)
    Wd = to_dev(W)
    for mode, iters in (("4o6", 0), ("soar", 3)):
        a = run(W, mode, iters, dev_W=Wd)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            b = run(W, mode, iters, dev_W=Wd)
        torch.cuda.synchronize()
        for k in ("codes", "scales"):
            assert np.array_equal(a[k], b[k])
        assert f32_bits(a["alpha"]) == f32_bits(b["alpha"])


def test_plain_entry_point_matches_ex():
    W = synth.normal_bf16(64, 512, seed=9)
    Wd = to_dev(W)
    L = nv.lib()
    for mode in range(4):
        codes = torch.empty((64, 256), dtype=torch.uint8, device="cuda")
        scales = torch.empty((64, 32), dtype=torch.uint8, device="cuda")
        alpha = torch.empty(1, dtype=torch.float32, device="cuda")
        say(f"plain nvfp4_quantize mode={mode}")
        st = L.nvfp4_quantize(Wd.data_ptr(), 64, 512, mode, 2, codes.data_ptr(), scales.data_ptr(), alpha.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        name = ["max", "4o6", "cjso", "soar"][mode]
        r = run(W, name, 2, dev_W=Wd)
        assert np.array_equal(codes.cpu().numpy(), r["codes"]) and np.array_equal(scales.cpu().numpy(), r["scales"])


def test_f32_entry_point_matches_oracle():
    """nvfp4_quantize_f32 (the plain binary32 entry point) with valid arguments, every mode, against the
    oracle bit for bit."""
    W = synth.normal_f32(48, 1040, seed=14)
    W[3, 5] *= 40.0  # an outlier sets alpha
    Wd = to_dev(W)
    L = nv.lib()
    for mode, name in enumerate(["max", "4o6", "cjso", "soar"]):
        codes = torch.empty((48, 520), dtype=torch.uint8, device="cuda")
        scales = torch.empty((48, 65), dtype=torch.uint8, device="cuda")
        alpha = torch.empty(1, dtype=torch.float32, device="cuda")
        say(f"plain nvfp4_quantize_f32 mode={mode}")
        st = L.nvfp4_quantize_f32(Wd.data_ptr(), 48, 1040, mode, 3, codes.data_ptr(), scales.data_ptr(),
                                  alpha.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        r = oracle.quantize(W, name, 3)
        assert np.array_equal(codes.cpu().numpy(), r["codes"]) and np.array_equal(scales.cpu().numpy(), r["scales"])
        assert f32_bits(float(alpha.cpu()[0])) == f32_bits(r["alpha"])


def test_graph_capture_replays_match_eager():
    W = synth.c2(1, rows=256, cols=1024)
    Wd = to_dev(W)
    outs = {m: (torch.empty((256, 512), dtype=torch.uint8, device="cuda"),
                torch.empty((256, 64), dtype=torch.uint8, device="cuda"),
                torch.empty(1, dtype=torch.float32, device="cuda"),
                torch.empty(nv.workspace_bytes(256, 1024, m), dtype=torch.uint8, device="cuda"))
            for m in ("max", "4o6", "cjso", "soar")}
    eager = {m: run(W, m, 4 if m in ("cjso", "soar") else 0, dev_W=Wd) for m in outs}

    def step():
        for m, (c, s, a, ws) in outs.items():
            nv.quantize(Wd, m, 4 if m in ("cjso", "soar") else 0, codes=c, scales=s, alpha=a, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("capturing graph")
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for c, s_, a, _ in outs.values():
            c.zero_(); s_.zero_(); a.zero_()
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for m, (c, s_, a, _) in outs.items():
            assert np.array_equal(c.cpu().numpy(), eager[m]["codes"]), (rep, m)
            assert np.array_equal(s_.cpu().numpy(), eager[m]["scales"]), (rep, m)
            assert f32_bits(float(a.cpu()[0])) == f32_bits(eager[m]["alpha"])
        run(W, "max", 0, dev_W=Wd)  # eager work between replays


def test_stage_events():
    W = synth.normal_bf16(128, 1024, seed=10)
    Wd = to_dev(W)
    n = nv.kernel_count("soar", 3)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    nv.quantize(Wd, "soar", 3, stage_events=ev)
    torch.cuda.synchronize()
    t = [ev[j].elapsed_time(ev[j + 1]) for j in range(n)]
    assert len(t) == 6 and all(x >= 0 for x in t)
    # NULL entries are skipped: a span over the three rounds, same outputs as without events
    sparse = [None] * (n + 1)
    sparse[2], sparse[5] = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c1, s1, a1 = nv.quantize(Wd, "soar", 3, stage_events=sparse)
    c0, s0, a0 = nv.quantize(Wd, "soar", 3)
    torch.cuda.synchronize()
    assert sparse[2].elapsed_time(sparse[5]) >= 0
    assert torch.equal(c0, c1) and torch.equal(s0, s1) and torch.equal(a0, a1)


# ------------------------------------------------------------------------------ codec kernels

def test_encode_e2m1_matches_oracle():
    x = [(np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)).view(np.float32)]
    for v in list(indep.GRID) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.0]:
        c = np.float32(v).view(np.uint32)
        nb = (np.arange(-4096, 4097, dtype=np.int64) + int(c)).astype(np.uint32).view(np.float32)
        x += [nb, -nb]
    g = np.random.default_rng(12)
    x.append(g.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32))
    x.append(np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-45, -1e-45, 3.4e38], np.float32))
    x = np.concatenate(x)[:-3]  # odd length: exercises the tail path
    say(f"encode_e2m1 n={x.size}")
    got = nv.encode_e2m1(torch.from_numpy(x).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.e2m1_codes(x))


def test_encode_e2m1_exhaustive():
    """Every binary32 bit pattern (2^32, in 16 chunks) through nvfp4_encode_e2m1, against a threshold
    encoder written with torch's own elementwise operations: magnitude index = number of thresholds
    passed (0.25 <, 0.75 <=, 1.25 <, 1.75 <=, 2.5 <, 3.5 <=, 5 <: nearest value, ties to the even code,
    saturating at 6; NaN passes none), sign bit only on nonzero codes."""
    chunk = 1 << 28
    for c in range(16):
        lo = c * chunk
        say(f"encode_e2m1 exhaustive chunk {c}/16")
        bits = torch.arange(lo, lo + chunk, dtype=torch.int64, device="cuda")
        bits = torch.where(bits >= 1 << 31, bits - (1 << 32), bits).to(torch.int32)
        x = bits.view(torch.float32)
        got = nv.encode_e2m1(x)
        a = x.abs()
        idx = (a > 0.25).to(torch.uint8)
        for t, strict in ((0.75, False), (1.25, True), (1.75, False), (2.5, True), (3.5, False), (5.0, True)):
            idx += (a > t) if strict else (a >= t)
        neg = torch.signbit(x) & (idx > 0)
        want = idx | (neg.to(torch.uint8) << 3)
        bad = torch.nonzero(got != want)
        assert bad.numel() == 0, f"chunk {c}: {bad.numel()} mismatches, first bits {int(bits[bad[0, 0]]) & 0xFFFFFFFF:#x}"
        del bits, x, got, a, idx, neg, want
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["4o6", "soar"])
def test_dequantize_matches_oracle(mode):
    W = synth.normal_bf16(96, 512, seed=13)
    Wd = to_dev(W)
    codes, scales, alpha = nv.quantize(Wd, mode, 2)
    exact = oracle.dequantize(codes.cpu().numpy(), scales.cpu().numpy(), float(alpha.cpu()[0]), 96, 512)
    f32 = nv.dequantize(codes, scales, alpha, torch.float32).cpu().numpy()
    assert np.array_equal(f32, exact.astype(np.float32))
    bf = nv.dequantize(codes, scales, alpha, torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    m, e = np.frexp(exact)
    e = np.maximum(e, -125)
    ref = np.ldexp(np.rint(np.ldexp(exact, 8 - e)), e - 8).astype(np.float32)  # nearest 8-bit significand
    assert np.array_equal(bf, (ref.view(np.uint32) >> 16).astype(np.uint16))


# ------------------------------------------------------------- windowed search vs the full scan

def coarse_bf16(seed, rows=64, cols=256):
    """Few distinct magnitudes (multiples of 2^-8 up to 3 * 2^-6) and many zeros: errors of different
    candidates often tie exactly."""
    g = np.random.default_rng(seed)
    v = g.integers(-3, 4, size=(rows, cols)).astype(np.float32)
    v *= g.choice([1.0, 0.5, 0.25], size=(rows, cols)).astype(np.float32)
    v[g.random((rows, cols)) < g.uniform(0.2, 0.9)] = 0
    v *= np.float32(2.0 ** -6)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def sparse_bf16(seed, rows=64, cols=256):
    """One to three small odd integers per block times a power of two."""
    g = np.random.default_rng(1000 + seed)
    v = np.zeros((rows * cols // 16, 16), np.float32)
    for i in range(v.shape[0]):
        n = int(g.integers(1, 4))
        pos = g.choice(16, size=n, replace=False)
        v[i, pos] = g.choice([1, 2, 3, 5, 6, 7, 9, 11, 13], size=n) * g.choice([-1, 1], size=n)
    v *= np.float32(2.0 ** int(g.integers(-9, -3)))
    v = v.reshape(rows, cols)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


WINDOW_CASES = {
    "c2_4096x4096": lambda: synth.c2(0),
    "c3_up_14336x4096": lambda: synth.c3(0, 0),
    "c5_l0_down_4096x11008": lambda: synth.c5(0, "down"),
    "on_grid": lambda: indep.on_grid_matrix(64, 256, -10, 7)[0],
    "on_grid_tiny_alpha": lambda: indep.on_grid_matrix(64, 256, -120, 3)[0],
    "coarse_0": lambda: coarse_bf16(0),
    "coarse_1": lambda: coarse_bf16(1),
    "sparse_0": lambda: sparse_bf16(0),
    "sparse_1": lambda: sparse_bf16(1),
    "ragged_3x48": lambda: synth.normal_bf16(3, 48, 5),
    # fp32 input: the same window with binary64 block sums
    "c1_fp32": lambda: synth.c1(0),
    "c2_widened_fp32": lambda: np.ascontiguousarray(indep.as_f32(synth.c2(0))),
    "normal_fp32": lambda: synth.normal_f32(512, 2048, seed=7),
    "coarse_fp32": lambda: np.ascontiguousarray(indep.as_f32(coarse_bf16(2))),
    "sparse_fp32": lambda: np.ascontiguousarray(indep.as_f32(sparse_bf16(2))),
    "ragged_fp32_3x48": lambda: synth.normal_f32(3, 48, seed=5),
}


@functools.lru_cache(maxsize=1)
def window_input(name):
    return WINDOW_CASES[name]()


@pytest.mark.parametrize("iters", [0, 2, 8])
@pytest.mark.parametrize("name", list(WINDOW_CASES))
def test_soar_window_equals_full_search(name, iters):
    """The default search (two or three quantise scales per reconstruct scale) and the 202-candidate
    scan give the same codes and scales on every block."""
    W = window_input(name)
    Wd = to_dev(W)
    a = run(W, "soar", iters, dev_W=Wd)
    b = run(W, "soar", iters, dev_W=Wd, full_search=True)
    assert f32_bits(a["alpha"]) == f32_bits(b["alpha"])
    diff = ~(np.all(a["codes"].reshape(-1, 8) == b["codes"].reshape(-1, 8), axis=1)
             & (a["scales"].reshape(-1) == b["scales"].reshape(-1)))
    assert not diff.any(), f"{diff.sum()} blocks differ, first {np.flatnonzero(diff)[:5]}"


@pytest.mark.parametrize("gen", [coarse_bf16, sparse_bf16])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_soar_tie_prone_inputs_match_oracle(gen, seed):
    W = gen(seed)
    compare_live(W, "soar", 8)
    compare_live(np.ascontiguousarray(indep.as_f32(W)), "soar", 8)  # the same values as fp32 input


@pytest.mark.parametrize("seed,rows,cols", [(0, 8, 256), (1, 64, 1024)])
def test_soar_exact_tie_blocks_match_oracle(seed, rows, cols):
    """fp32 blocks whose search ends in an exact tie between the two reconstruct scales, below the
    incumbent (synth.soar_tie_matrix; tests/test_oracle_soar_tie.py shows they are): the windowed search
    takes its equal-error branch there, and it and the full scan keep the first candidate in scan order."""
    W, kinds = synth.soar_tie_matrix(seed, rows, cols)
    say(f"tie blocks: {kinds.count('A')} A, {kinds.count('B')} B")
    compare_live(W, "soar", 0)
    g = run(W, "soar", 0, full_search=True)
    assert_exact(g, oracle.quantize(W, "soar", 0), "soar")


def band_restart_model(W, r):
    """binary32 model of the search's path choice: per block, whether its other reconstruct scale has a band
    candidate (s_k within 2^-20 of s_d) whose scaled weights fail the 32-ulp test while the incumbent's pass the
    8-ulp one (so the search certifies the incumbent, then walks the band window in k order); and the band
    candidate's scale."""
    alpha = np.float32(r["alpha"])
    w = W.reshape(-1, 16).astype(np.float32)
    dc = r["scales"].reshape(-1).astype(np.int64)
    br = np.array([oracle.e4m3_bracket(v) for v in r["dstar"].reshape(-1)])
    lo, hi = br[:, 0], br[:, 1]
    ev = np.array([oracle.e4m3_value(int(c)) for c in range(127)], np.float32)
    f = np.array([oracle.search_multiplier(k) for k in range(101)], np.float32)
    pair = (dc > 0) & (lo != hi) & ((dc == lo) | (dc == hi))
    vc, vo = ev[dc], ev[np.where(dc == lo, hi, lo)]

    def far(x, margin):
        u = x.view(np.uint32).astype(np.uint64)
        return (((u + margin) << 11) & 0xFFFFFFFF).min(1) >= ((2 * margin + 1) << 11)

    with np.errstate(divide="ignore"):
        xc = (w * (np.float32(1) / (alpha * vc).astype(np.float32))[:, None]).astype(np.float32)
        s = (alpha * (vc[:, None] * f[None, :]).astype(np.float32)).astype(np.float32)
        in_band = np.abs(np.float64(alpha) * vo.astype(np.float64)[:, None] / s.astype(np.float64) - 1) <= 2.0 ** -20
        sb = s[np.arange(len(s)), in_band.argmax(1)]
        xb = (w * (np.float32(1) / sb)[:, None]).astype(np.float32)
    band = pair & in_band.any(1)
    return band & far(xc, 8) & ~far(xb, 32), band, sb


def band_restart_rows(seed: int):
    """fp32 rows whose search walks band windows in k order. Rows 8..15 are scaled by 1/64 (normal E4M3 scales,
    a negligible share of alpha's sums). In each of their band blocks one element is set 3 binary32 ulps from
    fl(1.75 s_b), s_b the band scale, on the side that puts its scaled value x_b and its quotient u = |w| / s_d
    on opposite sides of the decision point 1.75: the band candidate's code for it is then not the nearest one,
    and its 32-ulp test fails. The oracle is run again and the elements placed again, three times, until alpha
    no longer moves."""
    W = synth.student_t(synth.rng(seed, 11), 4.0, (16, 4096), 0.02).astype(np.float32)
    W[8:] *= np.float32(1.0 / 64)
    wb = W.reshape(-1, 16)
    probe = np.arange(wb.shape[0]) >= wb.shape[0] // 2
    slot = {}
    for _ in range(3):
        r = oracle.quantize(W, "soar", 3)
        _, band, sb = band_restart_model(W, r)
        alpha = np.float64(np.float32(r["alpha"]))
        dc, dstar = r["scales"].reshape(-1), r["dstar"].reshape(-1)
        for i in np.flatnonzero(band & probe):
            lo, hi = oracle.e4m3_bracket(dstar[i])
            sd = alpha * oracle.e4m3_value(int(hi if dc[i] == lo else lo))
            up = sd > np.float64(sb[i])  # u = x_b s_b / s_d: below x_b when s_d > s_b
            k = slot.setdefault(i, (int(np.argmax(np.abs(wb[i]))) + 1) % 16)
            t = np.float32(1.75) * sb[i]
            for _ in range(3):
                t = np.nextafter(t, np.float32(np.inf) if up else np.float32(0), dtype=np.float32)
            wb[i, k] = np.copysign(t, wb[i, k] if wb[i, k] != 0 else np.float32(1))
    return W


def test_soar_band_windows_walked_in_order_match_oracle():
    """The search's band candidates whose codes cannot be certified: those lanes walk their three-candidate window
    in k order after the other lanes' first candidate. The rows are built so that over a hundred blocks take that
    path (the binary32 model says which; seeded workload rows almost never do), and so that in at least twenty of
    them the other scale wins with codes that differ from the band candidate's: a search that took an uncertified
    band candidate as its answer would get those blocks wrong."""
    W = band_restart_rows(3)
    r = oracle.quantize(W, "soar", 3)
    walked, band, sb = band_restart_model(W, r)
    xb = (W.reshape(-1, 16) * (np.float32(1) / sb)[:, None]).astype(np.float32)
    band_codes = oracle.e2m1_codes(xb.reshape(-1)).reshape(-1, 16)
    out_codes = oracle.unpack_codes(r["codes"]).reshape(-1, 16)
    br = np.array([oracle.e4m3_bracket(v) for v in r["dstar"].reshape(-1)])
    dc = oracle.quantize(W, "cjso", 3)["scales"].reshape(-1)  # the search's incumbent scales
    other_won = r["scales"].reshape(-1) == np.where(dc == br[:, 0], br[:, 1], br[:, 0])
    telling = walked & other_won & np.any(band_codes != out_codes, axis=1)
    say(f"band lanes {int(band.sum())}, walked in order {int(walked.sum())}, telling {int(telling.sum())}")
    assert walked.sum() >= 100 and telling.sum() >= 20
    g = run(W, "soar", 3)
    assert_exact(g, r, "soar")
    f = run(W, "soar", 3, full_search=True)
    assert_exact(f, r, "soar")


# ------------------------------------------------------------------- CJSO / SOAR from FourOverSix

INIT_CASES = {
    "c1_fp32": lambda: synth.c1(0),
    "ragged_3x48": lambda: synth.normal_bf16(3, 48, 5),
    "c2_rows": lambda: synth.c2(0, 128, 1024),
    "c3_rows": lambda: synth.c3(0, 0)[:64],
    "on_grid": lambda: indep.on_grid_matrix(32, 256, -10, 7)[0],
}


@pytest.mark.parametrize("mode,iters", [("cjso", 0), ("cjso", 3), ("cjso", 8), ("soar", 0), ("soar", 8)])
@pytest.mark.parametrize("name", list(INIT_CASES))
def test_init_4o6_matches_oracle(name, mode, iters):
    W = INIT_CASES[name]()
    g = run(W, mode, iters, init="4o6")
    r = oracle.quantize(W, mode, iters, init="4o6")
    assert_tolerance(W, g, r)
    assert_exact(g, r, mode)


def test_init_4o6_zero_rounds_is_4o6():
    W = synth.c2(0, 256, 1024)
    a = run(W, "cjso", 0, init="4o6")
    b = run(W, "4o6", 0)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    assert f32_bits(a["alpha"]) == f32_bits(b["alpha"])


# ---------------------------------------------------------------- search grids and reconstruct rules

SEARCH_CASES = {
    "c1_fp32_rows": lambda: np.ascontiguousarray(synth.c1(0)[:64]),
    "ragged_3x48": lambda: synth.normal_bf16(3, 48, 5),
    "c2_rows": lambda: synth.c2(0, 64, 1024),
    "on_grid_tiny_alpha": lambda: indep.on_grid_matrix(32, 256, -120, 3)[0],
    "coarse_0": lambda: coarse_bf16(0),
    "sparse_1": lambda: sparse_bf16(1),
}
SEARCHES = [((50, 100, 101), "quant"), ((50, 100, 101), "lsq"), ((1, 4, 7), "cjso"), ((100, 200, 201), "cjso"),
            ((1, 1, 16), "lsq"), ((45, 100, 13), "quant"), ((12345, 16777213, 9), "cjso"),
            ((1, 20, 60), "lsq"),
            ((4473412, 4194304, 1024), "cjso")]  # steps of 2^-22 around 16/15: several candidates in a band window


@pytest.mark.parametrize("grid,rule", SEARCHES)
@pytest.mark.parametrize("name", list(SEARCH_CASES))
def test_search_variants_match_oracle(name, grid, rule):
    W = SEARCH_CASES[name]()
    iters = 3
    g = run(W, "soar", iters, grid=grid, dd_rule=rule)
    r = oracle.quantize_search(W, iters, grid=grid, dd_rule=rule)
    assert_exact(g, r, "soar")


@pytest.mark.parametrize("grid", [(1, 4, 7), (100, 200, 201), (12345, 16777213, 9), (1, 20, 60), (7, 7, 1),
                                  (4473412, 4194304, 1024)])
@pytest.mark.parametrize("name", ["c2_4096x4096", "coarse_1", "on_grid", "ragged_3x48"])
def test_search_grid_window_equals_full_scan(name, grid):
    """The windowed search stays exact on other grids: it only needs the multipliers to increase."""
    W = window_input(name)
    Wd = to_dev(W)
    a = run(W, "soar", 2, dev_W=Wd, grid=grid)
    b = run(W, "soar", 2, dev_W=Wd, grid=grid, full_search=True)
    assert f32_bits(a["alpha"]) == f32_bits(b["alpha"])
    diff = ~(np.all(a["codes"].reshape(-1, 8) == b["codes"].reshape(-1, 8), axis=1)
             & (a["scales"].reshape(-1) == b["scales"].reshape(-1)))
    assert not diff.any(), f"{diff.sum()} blocks differ, first {np.flatnonzero(diff)[:5]}"


def test_search_variant_with_init_4o6():
    W = synth.c2(0, 64, 512)
    g = run(W, "soar", 2, init="4o6", grid=(1, 4, 7), dd_rule="lsq")
    r = oracle.quantize_search(W, 2, init="4o6", grid=(1, 4, 7), dd_rule="lsq")
    assert_exact(g, r, "soar")


def test_pages_search_spelled_out_is_the_default():
    W = synth.c2(0, 64, 1024)
    a = run(W, "soar", 2)
    b = run(W, "soar", 2, grid=(50, 100, 101), dd_rule="cjso")
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


# ------------------------------------------------------------------------------ error statistics

STATS_CASES = {
    "c1_fp32_max": (lambda: synth.c1(0), "max", 0),
    "c1_fp32_4o6": (lambda: synth.c1(0), "4o6", 0),
    "c2_rows_soar": (lambda: synth.c2(0, 128, 1024), "soar", 8),
    "ragged_cjso": (lambda: synth.normal_bf16(3, 48, 5), "cjso", 3),
    "on_grid_max": (lambda: indep.on_grid_matrix(32, 256, -10, 7)[0], "max", 0),
    "c2_full_4o6": (lambda: synth.c2(0), "4o6", 0),
}


@pytest.mark.parametrize("name", list(STATS_CASES))
def test_error_stats_match_oracle(name):
    """nvfp4_error_stats against the oracle's MSE (exact sum of the binary64 differences) and a numpy
    histogram of the codes."""
    gen, mode, iters = STATS_CASES[name]
    W = gen()
    Wd = to_dev(W)
    codes, scales, alpha = nv.quantize(Wd, mode, iters)
    sse, hist = nv.error_stats(Wd, codes, scales, alpha)
    torch.cuda.synchronize()
    c, s_, a = codes.cpu().numpy(), scales.cpu().numpy(), float(alpha.cpu()[0])
    n = W.size
    ref = oracle.mse(W, c, s_, a) * n
    got = float(sse.cpu()[0])
    if ref == 0.0:
        assert got == 0.0
    else:
        assert abs(got - ref) <= 1e-12 * ref, (got, ref)
    nib = np.stack([c & 15, c >> 4], axis=-1).reshape(-1)
    assert np.array_equal(hist.cpu().numpy(), np.bincount(nib, minlength=16))


# -------------------------------------------------------------------------- full-size digests

def golden():
    with open(os.path.join(GOLDEN, "full_size.json")) as f:
        return json.load(f)


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


WORKLOADS = {
    "c2": lambda: synth.c2(0),
    "c3_up": lambda: synth.c3(0, 0),
    "c3_down": lambda: synth.c3(1, 0),
    **{f"c5_l{layer}_{m}": (lambda layer=layer, m=m: synth.c5(layer, m)) for layer in (0, 31) for m in synth.C5_ORDER},
}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_size(name):
    G = golden()[name]
    W = WORKLOADS[name]()
    assert sha(W) == G["input_sha256"], "input generator drifted"
    Wd = to_dev(W)
    for mode, exp in G["modes"].items():
        iters = exp.get("iters", 0)
        g = run(W, mode, iters, dev_W=Wd)
        assert "%08x" % f32_bits(g["alpha"]) == exp["alpha"], mode
        if mode == "soar":
            d = np.load(os.path.join(GOLDEN, exp["sample"]))
            blocks = d["blocks"]
            gc = g["codes"].reshape(-1, 8)[blocks]
            gs = g["scales"].reshape(-1)[blocks]
            same = np.all(gc == d["codes"], axis=1) & (gs == d["scales"])
            assert same.all(), f"{(~same).sum()} sampled blocks differ"
            # every block: the digests of the oracle's search over the whole matrix
            assert sha(g["codes"]) == exp["codes"] and sha(g["scales"]) == exp["scales"], "soar: a block differs"
            for vname, v in exp.get("search_variants", {}).items():
                gv = run(W, mode, iters, dev_W=Wd, grid=tuple(v["grid"]), dd_rule=v["dd_rule"])
                assert "%08x" % f32_bits(gv["alpha"]) == exp["alpha"], vname
                same = (np.all(gv["codes"].reshape(-1, 8)[blocks] == d[f"{vname}_codes"], axis=1)
                        & (gv["scales"].reshape(-1)[blocks] == d[f"{vname}_scales"]))
                assert same.all(), f"{vname}: {(~same).sum()} sampled blocks differ"
                assert sha(gv["codes"]) == v["codes_all"] and sha(gv["scales"]) == v["scales_all"], vname
            continue
        if mode == "cjso":
            # tolerance first (MSE), then bit-exactness through the digests
            mse = oracle.mse(W, g["codes"], g["scales"], g["alpha"])
            assert abs(mse - exp["mse"]) <= 1e-5 * exp["mse"]
        if mode == "4o6":
            assert int(g["mchoice"].sum()) == exp["m4_blocks"] == int(g["stats"][1])
        assert sha(g["codes"]) == exp["codes"], mode
        assert sha(g["scales"]) == exp["scales"], mode


def test_reciprocal_is_ieee_division():
    """The search's binary32 reciprocal (nvfp4_reciprocal_f32) against numpy's IEEE division: every
    mantissa at exponents across the fast range and just outside it, the range boundaries, specials,
    and random bit patterns."""
    mant = np.arange(1 << 23, dtype=np.uint32)
    parts = [((np.uint32(e + 127) << np.uint32(23)) | mant) for e in (-126, -125, -100, -40, -1, 0, 1, 40, 100, 124, 125, 126)]
    g = np.random.default_rng(11)
    parts.append(g.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32))
    parts.append(np.array([0x00000000, 0x80000000, 0x00000001, 0x007FFFFF, 0x7F7FFFFF, 0x7F800000, 0xFF800000,
                           0x7FC00000, 0x01000000, 0x00FFFFFF, 0x7E000000, 0x7DFFFFFF], dtype=np.uint32))
    bits = np.concatenate(parts)
    s = bits.view(np.float32)
    say(f"reciprocal: {s.size} values")
    got = nv.reciprocal_f32(torch.from_numpy(s).cuda()).cpu().numpy()
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        want = np.float32(1.0) / s
    same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    # outside the fast range the kernel divides; where the quotient is subnormal (s >= 2^126) that division
    # may flush it to zero, which is not the reciprocal under test
    sub = (want != 0) & (np.abs(want) < np.float32(2.0 ** -126))
    same |= sub & (got == 0)
    fast = (s >= np.float32(2.0 ** -125)) & (s < np.float32(2.0 ** 125))
    assert fast.sum() > 12 * (1 << 22)
    assert same.all(), f"{(~same).sum()} differ, first input bits {int(bits[np.flatnonzero(~same)[0]]):#x}"
