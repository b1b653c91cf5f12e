"""nvfp4_quantize_noalloc (the entry point that allocates nothing; its scratch is a fixed device array in
the library) against nvfp4_quantize_ex with a caller workspace, through the C ABI: every mode, bf16 and
fp32, two calls in a row of which the second is smaller, bit for bit (codes, scales, alpha, M=4 map and
stats). Also the host-side rejections (a workspace passed in, a SOAR call too large for the array)."""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_elem_amd as nv
import synth

pytestmark = pytest.mark.gpu

MODES = (("max", 0), ("4o6", 0), ("cjso", 3), ("soar", 3))


def say(msg):
    print(msg, flush=True)


def device_matrix(rows, cols, dtype, seed):
    W = synth.c2(seed, rows, cols)
    t = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).cuda()
    return t if dtype == torch.bfloat16 else t.float().contiguous()


def call(entry, W, mode, iters, workspace=None):
    rows, cols = W.shape
    dev = W.device
    out = dict(codes=torch.full((rows, cols // 2), 0xA5, dtype=torch.uint8, device=dev),
               scales=torch.full((rows, cols // 16), 0xA5, dtype=torch.uint8, device=dev),
               alpha=torch.full((1,), -1.0, dtype=torch.float32, device=dev),
               mchoice=torch.full((rows, cols // 16), 0xA5, dtype=torch.uint8, device=dev),
               stats=torch.full((4,), -1, dtype=torch.int32, device=dev))
    a = nv._Args()
    a.W = W.data_ptr()
    a.dtype = nv.DTYPES[W.dtype]
    a.rows, a.cols, a.mode, a.iters = rows, cols, nv.MODES[mode], iters
    a.codes_out, a.scales_out, a.alpha_out = out["codes"].data_ptr(), out["scales"].data_ptr(), out["alpha"].data_ptr()
    a.mchoice_out = out["mchoice"].data_ptr() if mode == "4o6" else None
    a.stats_out = out["stats"].data_ptr()
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    a.stream = torch.cuda.current_stream().cuda_stream
    fn = nv.lib().nvfp4_quantize_noalloc if entry == "noalloc" else nv.lib().nvfp4_quantize_ex
    fn.argtypes = [ctypes.POINTER(nv._Args)]
    fn.restype = ctypes.c_int
    st = fn(ctypes.byref(a))
    assert st == 0, nv.status_string(st)
    return out


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("mode,iters", MODES)
def test_noalloc_equals_ex_on_two_calls(mode, iters, dtype):
    for rows, cols, seed in ((1024, 2048, 1), (96, 272, 2)):  # the second call is smaller
        say(f"noalloc {mode} {dtype} {rows}x{cols}")
        W = device_matrix(rows, cols, dtype, seed)
        ws = torch.empty(nv.workspace_bytes(rows, cols, mode), dtype=torch.uint8, device="cuda")
        ref = call("ex", W, mode, iters, ws)
        got = call("noalloc", W, mode, iters)
        torch.cuda.synchronize()
        for k in ("codes", "scales", "stats") + (("mchoice",) if mode == "4o6" else ()):
            assert torch.equal(got[k], ref[k]), (k, rows, cols)
        assert got["alpha"].view(torch.int32).item() == ref["alpha"].view(torch.int32).item()


def test_noalloc_rejections():
    lib = nv.lib()
    lib.nvfp4_noalloc_scratch_bytes.restype = ctypes.c_size_t
    cap = lib.nvfp4_noalloc_scratch_bytes()
    assert cap == 16 << 20
    a = nv._Args()
    a.W = a.codes_out = a.scales_out = a.alpha_out = 0x100000
    a.rows, a.cols, a.mode, a.iters = 64, 256, 0, 0
    a.workspace, a.workspace_bytes = 0x100000, 1 << 20
    assert lib.nvfp4_quantize_noalloc(ctypes.byref(a)) == -1  # no workspace may be passed
    a.workspace, a.workspace_bytes = None, 0
    a.mode, a.iters = 3, 2
    a.rows, a.cols = 16384, 16384  # SOAR scratch: 2 bytes per block, 32 MiB here
    assert nv.workspace_bytes(16384, 16384, "soar") > cap
    assert lib.nvfp4_quantize_noalloc(ctypes.byref(a)) == -5
    assert "scratch" in nv.status_string(-5)
