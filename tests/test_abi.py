"""The HIP library loads, exports every function include/nvfp4.h declares, and rejects bad arguments on
the host before touching a device (CPU only: no call here passes validation)."""
import ctypes
import os
import re

import pytest

import nvfp4_block_scaled_elem_amd as nv
from nvfp4_block_scaled_elem_amd import build as nvbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, INVALID, SHAPE, WORKSPACE = 0, -1, -2, -3
FAKE = 0x100000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nv.LIB_PATH):
        nvbuild.build()
    return nv.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n


def args(**kw):
    a = nv._Args()
    a.W, a.dtype, a.rows, a.cols, a.mode, a.iters = FAKE, 0, 64, 256, 0, 0
    a.codes_out, a.scales_out, a.alpha_out = FAKE, FAKE, FAKE
    a.workspace, a.workspace_bytes = None, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,err", [
    (dict(W=None), INVALID), (dict(codes_out=None), INVALID), (dict(scales_out=None), INVALID),
    (dict(alpha_out=None), INVALID), (dict(rows=0), INVALID), (dict(cols=-16), INVALID),
    (dict(cols=24), SHAPE), (dict(rows=1 << 40, cols=1 << 20), SHAPE), (dict(rows=(1 << 31) + 1, cols=16), SHAPE),
    (dict(mode=4), INVALID),
    (dict(mode=-1), INVALID), (dict(dtype=2), INVALID), (dict(iters=-1), INVALID), (dict(iters=1001), INVALID),
    (dict(W=FAKE + 8), INVALID), (dict(codes_out=FAKE + 4), INVALID), (dict(alpha_out=FAKE + 2), INVALID),
    (dict(workspace=FAKE + 64, workspace_bytes=1 << 30), INVALID),
    (dict(workspace=FAKE, workspace_bytes=16), WORKSPACE),
    (dict(mode=3, iters=8, workspace=FAKE, workspace_bytes=1024), WORKSPACE),
    (dict(flags=4), INVALID), (dict(flags=0x80000000), INVALID), (dict(flags=2, mode=0), INVALID),
    (dict(flags=2, mode=1), INVALID),
    # search settings: SOAR only, valid grids and rules only (a valid one reaches the workspace check)
    (dict(mode=2, dd_rule=1), INVALID), (dict(mode=2, search_num0=1, search_den=2, search_count=3), INVALID),
    (dict(mode=3, dd_rule=3), INVALID), (dict(mode=3, dd_rule=-1), INVALID),
    (dict(mode=3, search_num0=0, search_den=100, search_count=101), INVALID),
    (dict(mode=3, search_num0=50, search_den=0, search_count=101), INVALID),
    (dict(mode=3, search_num0=50, search_den=100, search_count=0), INVALID),
    (dict(mode=3, search_num0=50, search_den=100, search_count=1025), INVALID),
    (dict(mode=3, search_num0=1, search_den=1, search_count=17), INVALID),
    (dict(mode=3, search_num0=1, search_den=(1 << 24) + 1, search_count=1), INVALID),
    (dict(mode=3, search_num0=1, search_den=2, search_count=3, workspace=FAKE, workspace_bytes=16), WORKSPACE),
    (dict(mode=3, search_num0=1, search_den=1, search_count=16, dd_rule=2, workspace=FAKE, workspace_bytes=16),
     WORKSPACE),
])
def test_quantize_ex_rejects(L, kw, err):
    a = args(**kw)
    assert L.nvfp4_quantize_ex(ctypes.byref(a)) == err


def test_quantize_ex_null_args(L):
    assert L.nvfp4_quantize_ex(None) == INVALID


def test_stage_events_count_checked(L):
    ev = (ctypes.c_void_p * 2)(FAKE, FAKE)
    a = args(mode=2, iters=3)
    a.stage_events = ctypes.cast(ev, ctypes.c_void_p)
    a.n_stage_events = 2
    assert L.nvfp4_quantize_ex(ctypes.byref(a)) == INVALID


def test_plain_entry_points_reject(L):
    assert L.nvfp4_quantize(None, 4, 16, 0, 0, FAKE, FAKE, FAKE, None) == INVALID
    assert L.nvfp4_quantize(FAKE, 4, 17, 0, 0, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.nvfp4_quantize_f32(FAKE, 4, 16, 9, 0, FAKE, FAKE, FAKE, None) == INVALID
    assert L.nvfp4_encode_e2m1(None, 10, FAKE, None) == INVALID
    assert L.nvfp4_encode_e2m1(FAKE, 10, FAKE + 1, None) == INVALID
    assert L.nvfp4_encode_e2m1(FAKE, 0, FAKE, None) == OK  # nothing to do
    assert L.nvfp4_reciprocal_f32(None, 10, FAKE, None) == INVALID
    assert L.nvfp4_reciprocal_f32(FAKE, 10, FAKE + 2, None) == INVALID
    assert L.nvfp4_reciprocal_f32(FAKE, (1 << 35) + 1, FAKE, None) == SHAPE
    assert L.nvfp4_reciprocal_f32(FAKE, 0, FAKE, None) == OK
    assert L.nvfp4_encode_e2m1(FAKE, (1 << 35) + 1, FAKE, None) == SHAPE
    assert L.nvfp4_dequantize(FAKE, FAKE, FAKE, 4, 24, FAKE, 0, None) == SHAPE
    assert L.nvfp4_dequantize(FAKE, FAKE, FAKE, 4, 32, FAKE, 3, None) == INVALID
    assert L.nvfp4_dequantize(FAKE, FAKE, FAKE, 4, 32, FAKE + 8, 1, None) == INVALID


def test_error_stats_rejects(L):
    f = L.nvfp4_error_stats
    assert f(None, 0, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 2, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 0, 4, 24, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 0, 0, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE + 8, 0, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 0, 4, 16, FAKE, FAKE, FAKE, FAKE + 4, FAKE, None) == INVALID
    assert f(FAKE, 1, 4, 16, FAKE, FAKE, FAKE, FAKE, None, None) == INVALID


def test_matmul_rejects(L):
    f = L.nvfp4_matmul
    assert f(None, 1, 32, FAKE, FAKE, FAKE, 8, FAKE, 0, None) == INVALID
    assert f(FAKE, 0, 32, FAKE, FAKE, FAKE, 8, FAKE, 0, None) == INVALID
    assert f(FAKE, 1, 32, FAKE, FAKE, FAKE, 0, FAKE, 0, None) == INVALID
    assert f(FAKE, 1, 32, FAKE, FAKE, FAKE, 8, FAKE, 2, None) == INVALID  # output dtype
    assert f(FAKE, 1, 24, FAKE, FAKE, FAKE, 8, FAKE, 0, None) == SHAPE  # K % 16
    assert f(FAKE, 1, 16, FAKE, FAKE, FAKE, (1 << 25) + 1, FAKE, 0, None) == SHAPE
    assert f(FAKE, 1 << 20, 16, FAKE, FAKE, FAKE, 1 << 19, FAKE, 0, None) == SHAPE  # 2^24 tiles
    assert f(FAKE + 8, 1, 32, FAKE, FAKE, FAKE, 8, FAKE, 0, None) == INVALID  # alignment
    assert f(FAKE, 1, 32, FAKE + 8, FAKE, FAKE, 8, FAKE, 0, None) == INVALID
    assert f(FAKE, 1, 32, FAKE, FAKE, FAKE + 2, 8, FAKE, 0, None) == INVALID
    assert f(FAKE, 1, 32, FAKE, FAKE, FAKE, 8, FAKE + 8, 0, None) == INVALID


def test_matmul_ex_rejects(L):
    f = L.nvfp4_matmul_ex
    assert f(None, 1, 32, FAKE, FAKE, FAKE, 8, FAKE, 0, None, 0, None) == INVALID
    assert f(FAKE, 1, 24, FAKE, FAKE, FAKE, 8, FAKE, 0, None, 0, None) == SHAPE
    # K split at 1024 x 1024 x 256: too small a workspace, a misaligned one
    need = L.nvfp4_matmul_workspace_bytes(1024, 1024, 256)
    assert need > 0
    assert f(FAKE, 1024, 1024, FAKE, FAKE, FAKE, 256, FAKE, 0, FAKE, need - 1, None) == WORKSPACE
    assert f(FAKE, 1024, 1024, FAKE, FAKE, FAKE, 256, FAKE, 0, FAKE + 16, need, None) == INVALID
    plan = (ctypes.c_int64 * 10)()
    assert L.nvfp4_matmul_plan(1024, 1024, 256, None) == INVALID
    assert L.nvfp4_matmul_plan(1024, 1000, 256, ctypes.cast(plan, ctypes.c_void_p)) == INVALID
    assert L.nvfp4_matmul_plan(1024, 1024, 256, ctypes.cast(plan, ctypes.c_void_p)) == OK
    assert plan[9] == need


def test_sizes_and_counts(L):
    assert L.nvfp4_workspace_bytes(4096, 4096, 0) > 0
    assert L.nvfp4_workspace_bytes(4096, 4096, 3) >= L.nvfp4_workspace_bytes(4096, 4096, 2) + 2 * 4096 * 256
    assert L.nvfp4_workspace_bytes(4096, 4095, 0) == 0
    assert L.nvfp4_workspace_bytes(4096, 4096, 5) == 0
    assert [L.nvfp4_kernel_count(m, 8) for m in range(4)] == [2, 2, 10, 11]
    assert L.nvfp4_kernel_count(2, 0) == 2 and L.nvfp4_kernel_count(3, 0) == 3
    assert L.nvfp4_kernel_count(7, 0) == -1 and L.nvfp4_kernel_count(2, -1) == -1


def test_status_strings(L):
    for s in (OK, INVALID, SHAPE, WORKSPACE, -4, 99):
        assert isinstance(nv.status_string(s), str) and nv.status_string(s)


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(nv.NVFP4Error):
        nv.quantize(torch.zeros(4, 16, dtype=torch.bfloat16), "max")


def test_args_struct_layout_matches_header(tmp_path):
    """The binding's ctypes struct has the C compiler's size and field offsets for nvfp4_args_t."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = [f for f, _ in nv._Args._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"nvfp4.h\"\nint main(void) {\n"
                   + 'printf("%zu\\n", sizeof(nvfp4_args_t));\n'
                   + "".join(f'printf("%zu\\n", offsetof(nvfp4_args_t, {f}));\n' for f in fields)
                   + "return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(nv._Args)
    assert out[1:] == [getattr(nv._Args, f).offset for f in fields]


def test_gptq_rejects(L):
    f = L.nvfp4_gptq
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_void_p]

    def call(W=FAKE, dtype=0, rows=64, cols=256, H=FAKE, damp=0.01, codes=FAKE, scales=FAKE, alpha=FAKE, ws=None,
             wsb=0):
        return f(W, dtype, rows, cols, H, damp, codes, scales, alpha, ws, wsb, None)

    assert call(W=None) == INVALID and call(H=None) == INVALID and call(codes=None) == INVALID
    assert call(scales=None) == INVALID and call(alpha=None) == INVALID
    assert call(rows=0) == INVALID and call(cols=-16) == INVALID and call(dtype=2) == INVALID
    assert call(damp=-0.01) == INVALID and call(damp=float("nan")) == INVALID and call(damp=float("inf")) == INVALID
    assert call(cols=24) == SHAPE and call(cols=32784) == SHAPE
    assert call(rows=(1 << 32) // 256 + 1) == SHAPE and call(rows=65535 * 64 + 1, cols=16) == SHAPE
    assert call(W=FAKE + 8) == INVALID and call(H=FAKE + 4) == INVALID and call(codes=FAKE + 4) == INVALID
    assert call(alpha=FAKE + 2) == INVALID and call(ws=FAKE + 64, wsb=1 << 30) == INVALID
    assert call(ws=FAKE, wsb=1024) == WORKSPACE


def test_gptq_workspace_bytes(L):
    f = L.nvfp4_gptq_workspace_bytes
    f.argtypes = [ctypes.c_int64, ctypes.c_int64]
    f.restype = ctypes.c_size_t
    assert f(4096, 4096) >= 8 * (4096 * 4096 + 4096 * 4096)
    assert f(4096, 4095) == 0 and f(0, 16) == 0 and f(16, 32784) == 0
