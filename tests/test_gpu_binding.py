"""The Python binding checks every caller-supplied buffer before it calls the C ABI (the kernels write
through bare pointers): too small, wrong dtype or wrong device raises NVFP4Error and launches nothing;
larger buffers are accepted and give the same results as the binding's own allocations."""
import pytest
import torch

import nvfp4_block_scaled_elem_amd as nv
import synth

pytestmark = pytest.mark.gpu

ROWS, COLS = 64, 256


@pytest.fixture(scope="module")
def W():
    return torch.from_numpy(synth.normal_bf16(ROWS, COLS, 3).view("int16")).view(torch.bfloat16).cuda()


def u8(n):
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


BAD_BUFFERS = {  # built lazily: collection must not touch the GPU
    "codes_short": lambda: dict(codes=u8(ROWS * COLS // 2 - 1)),
    "codes_int16": lambda: dict(codes=torch.zeros(ROWS * COLS // 4, dtype=torch.int16, device="cuda")),
    "scales_short": lambda: dict(scales=u8(ROWS * COLS // 16 - 1)),
    "alpha_f64": lambda: dict(alpha=torch.zeros(1, dtype=torch.float64, device="cuda")),
    "alpha_empty": lambda: dict(alpha=torch.zeros(0, dtype=torch.float32, device="cuda")),
    "mchoice_short": lambda: dict(mchoice=u8(ROWS * COLS // 16 - 8)),
    "stats_short": lambda: dict(stats=torch.zeros(3, dtype=torch.int32, device="cuda")),
    "codes_strided": lambda: dict(codes=u8(ROWS * COLS)[::2]),
    "codes_host": lambda: dict(codes=torch.zeros(ROWS * COLS // 2, dtype=torch.uint8)),
}


@pytest.mark.parametrize("case", sorted(BAD_BUFFERS))
def test_quantize_rejects_bad_buffers(W, case):
    with pytest.raises(nv.NVFP4Error):
        nv.quantize(W, "4o6", **BAD_BUFFERS[case]())


def test_quantize_rejects_unknown_mode(W):
    with pytest.raises(nv.NVFP4Error):
        nv.quantize(W, "nearest")


def test_larger_buffers_give_the_same_results(W):
    ref_c, ref_s, ref_a = nv.quantize(W, "soar", 2)
    codes, scales = u8(ROWS * COLS // 2 + 64), u8(ROWS * COLS // 16 + 64)
    codes[ROWS * COLS // 2:] = 0xAB
    stats = torch.zeros(8, dtype=torch.int32, device="cuda")
    ws = torch.zeros(nv.workspace_bytes(ROWS, COLS, "soar") // 4 + 64, dtype=torch.int32, device="cuda")
    c, s, a = nv.quantize(W, "soar", 2, codes=codes, scales=scales, stats=stats, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(c[:ROWS * COLS // 2].view(ROWS, -1), ref_c)
    assert torch.equal(s[:ROWS * COLS // 16].view(ROWS, -1), ref_s)
    assert torch.equal(a, ref_a)
    assert bool((codes[ROWS * COLS // 2:] == 0xAB).all())  # nothing written past the matrix


def test_dequantize_and_stats_and_matmul_reject_short_buffers(W):
    c, s, a = nv.quantize(W, "max")
    with pytest.raises(nv.NVFP4Error):
        nv.dequantize(c, s[:-1], a)
    with pytest.raises(nv.NVFP4Error):
        nv.dequantize(c.reshape(-1), s, a)
    with pytest.raises(nv.NVFP4Error):
        nv.dequantize(c, s, a.double())
    with pytest.raises(nv.NVFP4Error):
        nv.error_stats(W, c[:-1], s, a)
    X = torch.zeros(4, COLS, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.NVFP4Error):
        nv.matmul(X, c, s.reshape(-1)[:-16], a)
    with pytest.raises(nv.NVFP4Error):
        nv.matmul(X, c, s, a.double())
