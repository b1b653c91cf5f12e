"""GPU GPTQ (FourOverSix frame fixed first) against the oracle (oracle/gptq.py).

Both sides work in binary64 but by different algorithms: the oracle inverts H and applies the published
updates column by column; the kernels factor H once and accumulate the same sums in blocks. Their targets
differ by rounding only (relative ~1e-13 here), and a code could differ only where a target lies that
close to a rounding threshold, which none of these seeded cases does. So codes, scales and alpha are
compared exactly."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_elem_amd as nv
import synth
from oracle import gptq as og

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def dev_w(W):
    if W.dtype == np.uint16:
        return torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(W).cuda()


def run_gpu(W, H, percdamp=0.01, **kw):
    c, s, a = nv.gptq(dev_w(W), torch.from_numpy(H).cuda(), percdamp, **kw)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), float(a.cpu()[0])


CASES = [  # rows, cols, dead inputs, seed: ragged column blocks (cols % 64 != 0), rows % 64 != 0
    (5, 16, 0, 1), (3, 80, 0, 2), (70, 144, 5, 3), (130, 256, 0, 4), (257, 320, 2, 5), (64, 1040, 0, 6),
]


@pytest.mark.parametrize("rows,cols,dead,seed", CASES)
def test_gptq_matches_oracle(rows, cols, dead, seed):
    say(f"gptq {rows}x{cols} dead={dead} seed={seed}")
    W = synth.normal_bf16(rows, cols, seed)
    H = synth.hessian(cols, seed, dead=dead)
    ref = og.gptq(W, H, 0.01)
    c, s, a = run_gpu(W, H)
    assert a == ref["alpha"]
    assert np.array_equal(s, ref["scales"])
    assert np.array_equal(c, ref["codes"]), f"{np.sum(c != ref['codes'])} code bytes differ"


@pytest.mark.parametrize("percdamp", [0.0, 0.05, 1.0])
def test_gptq_damping(percdamp):
    say(f"gptq damping {percdamp}")
    W = synth.normal_bf16(40, 192, 7)
    H = synth.hessian(192, 7)
    ref = og.gptq(W, H, percdamp)
    c, s, a = run_gpu(W, H, percdamp)
    assert a == ref["alpha"] and np.array_equal(s, ref["scales"]) and np.array_equal(c, ref["codes"])


def test_gptq_fp32_weights():
    say("gptq fp32")
    W = synth.normal_f32(33, 208, 8)
    H = synth.hessian(208, 8)
    ref = og.gptq(W, H, 0.01)
    c, s, a = run_gpu(W, H)
    assert a == ref["alpha"] and np.array_equal(s, ref["scales"]) and np.array_equal(c, ref["codes"])


def test_gptq_caller_workspace_and_repeat():
    say("gptq workspace")
    W = synth.normal_bf16(50, 128, 9)
    H = synth.hessian(128, 9)
    ref = og.gptq(W, H, 0.01)
    ws = torch.empty(nv.gptq_workspace_bytes(50, 128) + 4096, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        c, s, a = run_gpu(W, H, workspace=ws)
        assert a == ref["alpha"] and np.array_equal(s, ref["scales"]) and np.array_equal(c, ref["codes"])
    W2 = synth.normal_bf16(20, 64, 10)
    H2 = synth.hessian(64, 10)
    ref2 = og.gptq(W2, H2, 0.01)
    c, s, a = run_gpu(W2, H2, workspace=ws)  # a smaller problem in the same workspace
    assert a == ref2["alpha"] and np.array_equal(c, ref2["codes"])


def test_gptq_indefinite_hessian_is_reported_in_band():
    say("gptq indefinite H")
    W = synth.normal_bf16(8, 64, 11)
    H = np.eye(64)
    H[5, 5] = -1.0  # not dead (nonzero), and the damping cannot make it positive
    c, s, a = run_gpu(W, H)
    assert np.isnan(a) and not c.any()


def test_gptq_rejects_bad_arguments():
    W = dev_w(synth.normal_bf16(8, 64, 12))
    with pytest.raises(nv.NVFP4Error):
        nv.gptq(W, torch.eye(64, device="cuda"))  # float32 H
    with pytest.raises(nv.NVFP4Error):
        nv.gptq(W, torch.eye(48, dtype=torch.float64, device="cuda"))
    with pytest.raises(nv.NVFP4Error):
        nv.gptq(W, torch.eye(64, dtype=torch.float64, device="cuda"), -1.0)


def test_gptq_full_size_sample():
    """4096 x 4096 bf16 (the attention-projection workload) with a 4096-input second moment: every 61st
    row against the oracle (rows are independent once H and the block scales are fixed)."""
    say("gptq full size 4096x4096")
    W = synth.c2(0)
    H = synth.hessian(4096, 0, n=4096)
    c, s, a = run_gpu(W, H)
    rows = np.arange(0, 4096, 61)
    ref = og.gptq(W, H, 0.01, rows=rows)
    assert a == ref["alpha"] and np.array_equal(s, ref["scales"])
    diff = np.sum(c[rows] != ref["codes"])
    assert diff == 0, f"{diff} code bytes differ"


def test_gptq_graph_replays_match_eager():
    """nvfp4_gptq with caller buffers captured in a graph (its kernels clear nothing with memsets),
    replayed three times with eager work in between: every replay equals the eager call."""
    say("gptq graph capture")
    W = dev_w(synth.normal_bf16(96, 320, 13))
    H = torch.from_numpy(synth.hessian(320, 13)).cuda()
    ws = torch.empty(nv.gptq_workspace_bytes(96, 320), dtype=torch.uint8, device="cuda")
    ref = [t.clone() for t in nv.gptq(W, H, workspace=ws)]
    torch.cuda.synchronize()
    outs = (torch.empty_like(ref[0]), torch.empty_like(ref[1]), torch.empty_like(ref[2]))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.gptq(W, H, codes=outs[0], scales=outs[1], alpha=outs[2], workspace=ws)
    for rep in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), rep
        nv.quantize(W, "max")  # eager work between replays
        torch.cuda.synchronize()


def test_gptq_mlp_shape_sample():
    """11008 x 4096 bf16 (an MLP up/gate projection of the 7B-shaped workload): every 97th row against
    the oracle."""
    say("gptq 11008x4096")
    W = synth.c5(0, "gate")
    H = synth.hessian(4096, 14, n=4096)
    c, s, a = run_gpu(W, H)
    rows = np.arange(0, W.shape[0], 97)
    ref = og.gptq(W, H, 0.01, rows=rows)
    assert a == ref["alpha"] and np.array_equal(s, ref["scales"])
    assert np.array_equal(c[rows], ref["codes"])


def test_gptq_long_rows_ragged_group():
    """cols = 6160: 96 full column blocks and a 16-column one, the last group of 4 blocks incomplete."""
    say("gptq 256x6160")
    W = synth.normal_bf16(256, 6160, 15)
    H = synth.hessian(6160, 15, n=4096)
    c, s, a = run_gpu(W, H)
    rows = np.arange(0, 256, 5)
    ref = og.gptq(W, H, 0.01, rows=rows)
    assert a == ref["alpha"] and np.array_equal(s, ref["scales"])
    assert np.array_equal(c[rows], ref["codes"])


@pytest.mark.parametrize("case", ["zero_w", "zero_h", "inf_w"])
def test_gptq_degenerate_inputs(case):
    """All-zero weights (alpha 0, every code 0), an all-zero H (every input dead: every weight counts as
    zero) and a weight that is infinite (FourOverSix's in-band result: alpha NaN, zero codes and scales),
    each against the oracle."""
    say(f"gptq degenerate {case}")
    W = synth.normal_bf16(24, 96, 16)
    H = synth.hessian(96, 16)
    if case == "zero_w":
        W = np.zeros_like(W)
    elif case == "zero_h":
        H = np.zeros_like(H)
    else:
        W = W.copy()
        W[3, 17] = 0x7F80  # +inf in bf16
    with np.errstate(all="ignore"):  # the oracle's sweep carries the infinity through its arithmetic
        ref = og.gptq(W, H, 0.01)
    c, s, a = run_gpu(W, H)
    assert np.array_equal(c, ref["codes"]) and np.array_equal(s, ref["scales"])
    assert (np.isnan(a) and np.isnan(ref["alpha"])) or a == ref["alpha"]
    if case != "inf_w":
        assert not c.any()
    else:
        assert np.isnan(a) and not c.any() and not s.any()
