"""Write the full-size expected outputs that the GPU parity tests compare against.

Every value here comes from the oracle (``oracle/``) run on the seeded inputs of ``synth``; nothing
comes from the GPU path. The oracle takes minutes at these sizes (CJSO(8) on a 14336 x 4096 matrix is
about two), too slow for a test, so this script runs it once and stores:
  * full_size.json: per workload, the SHA-256 of the input bytes, and per mode alpha (binary32 bits),
    the SHA-256 of the codes and of the scales, the FourOverSix M=4 block count and the MSE;
  * for SOAR, the SHA-256 of the codes and scales of every block (the oracle runs the search block by
    block from its own CJSO state; the blocks are shared out over the worker processes), and
    <workload>_soar_sample.npz, the expected codes and scales of a fixed sample of blocks, which tells
    how many blocks differ when a digest does not match; for the workloads in SEARCH_VARIANTS the same
    for other search grids and reconstruct-pair rules (keys <variant>_codes, <variant>_scales).

Run from the repository root:  python tests/golden/make_golden.py  [-j 8] [--only c2:soar ...]
(--only reruns the named jobs and keeps the other entries of full_size.json.)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

ITERS = 8
SOAR_SAMPLE_STRIDE = 127  # every 127th block: ~8k blocks of a 4096 x 4096 matrix


def workloads():
    return {
        "c2": lambda: synth.c2(0),
        "c3_up": lambda: synth.c3(0, 0),
        "c3_down": lambda: synth.c3(1, 0),
        **{f"c5_l{layer}_{m}": (lambda layer=layer, m=m: synth.c5(layer, m))
           for layer in (0, 31) for m in synth.C5_ORDER},
    }


# which modes are stored per workload (the configurations name them)
PLAN = {
    "c2": ["max", "4o6", "cjso", "soar"],
    "c3_up": ["4o6", "cjso"],
    "c3_down": ["4o6", "cjso"],
    # every matrix of the first layer in both of C5's modes, every matrix of the last layer in FourOverSix
    **{f"c5_l0_{m}": ["4o6", "soar"] for m in synth.C5_ORDER},
    **{f"c5_l31_{m}": ["4o6"] for m in synth.C5_ORDER},
}


# search variants stored beside the page's search: name -> ((num0, den, count), reconstruct-pair rule)
SEARCH_VARIANTS = {
    "c2": {"fine_lsq": ((100, 200, 201), "lsq"), "coarse_quant": ((1, 4, 7), "quant"),
           "wide_cjso": ((1, 20, 60), "cjso")},
}


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def f32_hex(x: float) -> str:
    return "%08x" % int(np.float32(x).view(np.uint32))


def sample_blocks(nblk: int) -> np.ndarray:
    return np.arange(0, nblk, SOAR_SAMPLE_STRIDE, dtype=np.int64)


def job(name: str, mode: str):
    W = workloads()[name]()
    out = {"input_sha256": sha(W), "shape": list(W.shape)}
    if mode in ("max", "4o6"):
        r = oracle.quantize(W, mode)
        out.update(alpha=f32_hex(r["alpha"]), codes=sha(r["codes"]), scales=sha(r["scales"]),
                   mse=oracle.mse(W, r["codes"], r["scales"], r["alpha"]))
        if mode == "4o6":
            out["m4_blocks"] = int(r["mchoice"].sum())
    elif mode == "cjso":
        r = oracle.quantize(W, "cjso", ITERS, trace=True)
        out.update(alpha=f32_hex(r["alpha"]), codes=sha(r["codes"]), scales=sha(r["scales"]),
                   alpha_trace=[f32_hex(a) for a in r["alpha_trace"]],
                   mse=oracle.mse(W, r["codes"], r["scales"], r["alpha"]))
    else:  # soar: CJSO state of the whole matrix, then the search on sampled blocks (every block: full_search)
        r = oracle.quantize(W, "cjso", ITERS)
        out["state"] = {"alpha": r["alpha"], "scales": r["scales"], "dstar": r["dstar"]}
        blocks = sample_blocks(r["scales"].size)
        c, s = oracle.soar_blocks(W, r["alpha"], r["scales"], r["dstar"], blocks)
        fname = f"{name}_soar_sample.npz"
        extra, variants = {}, {}
        for vname, (grid, rule) in SEARCH_VARIANTS.get(name, {}).items():
            vc, vs = oracle.soar_blocks(W, r["alpha"], r["scales"], r["dstar"], blocks, grid=grid, dd_rule=rule)
            extra[f"{vname}_codes"], extra[f"{vname}_scales"] = vc, vs
            variants[vname] = {"grid": list(grid), "dd_rule": rule, "codes": sha(vc), "scales": sha(vs)}
        np.savez_compressed(os.path.join(HERE, fname), blocks=blocks, codes=c, scales=s, **extra)
        out.update(alpha=f32_hex(r["alpha"]), sample=fname, sample_codes=sha(c), sample_scales=sha(s),
                   iters=ITERS)
        if variants:
            out["search_variants"] = variants
    if mode == "cjso":
        out["iters"] = ITERS
    return name, mode, out


_W_CACHE = {}


def search_chunk(name, alpha, scales, dstar, lo, hi, grid, rule):
    if name not in _W_CACHE:  # one workload per worker process at a time
        _W_CACHE.clear()
        _W_CACHE[name] = workloads()[name]()
    W = _W_CACHE[name]
    blocks = np.arange(lo, hi, dtype=np.int64)
    kw = {} if grid is None else {"grid": grid, "dd_rule": rule}
    return oracle.soar_blocks(W, alpha, scales, dstar, blocks, **kw)


def full_search(ex, name, st, grid, rule, jobs):
    """The oracle's search on every block from the CJSO state st, in contiguous chunks over the workers;
    codes [blocks][8] and scales in block order."""
    nblk = st["scales"].size
    step = (nblk + 4 * jobs - 1) // (4 * jobs)
    bounds = [(lo, min(lo + step, nblk)) for lo in range(0, nblk, step)]
    parts = list(ex.map(search_chunk, *zip(*[(name, st["alpha"], st["scales"], st["dstar"], lo, hi, grid, rule)
                                               for lo, hi in bounds])))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=4)
    ap.add_argument("--only", nargs="*", default=None, help="jobs as workload:mode")
    args = ap.parse_args()
    jobs = [(n, m) for n, modes in PLAN.items() for m in modes]
    result = {}
    if args.only:
        jobs = [j for j in jobs if f"{j[0]}:{j[1]}" in args.only]
        with open(os.path.join(HERE, "full_size.json")) as f:
            result = json.load(f)
    with ProcessPoolExecutor(max_workers=args.j) as ex:
        states = []
        for name, mode, out in ex.map(job, *zip(*jobs)):
            result.setdefault(name, {"modes": {}})
            result[name]["input_sha256"] = out.pop("input_sha256")
            result[name]["shape"] = out.pop("shape")
            if "state" in out:
                states.append((name, out.pop("state")))
            result[name]["modes"][mode] = out
            print(name, mode, out.get("alpha"), flush=True)
        for name, st in states:  # the search on every block, blocks shared out over the workers
            exp = result[name]["modes"]["soar"]
            c, s = full_search(ex, name, st, None, None, args.j)
            exp["codes"], exp["scales"] = sha(c), sha(s)
            for vname, v in exp.get("search_variants", {}).items():
                c, s = full_search(ex, name, st, tuple(v["grid"]), v["dd_rule"], args.j)
                v["codes_all"], v["scales_all"] = sha(c), sha(s)
            print(name, "soar, every block", exp["codes"][:12], flush=True)
    with open(os.path.join(HERE, "full_size.json"), "w") as f:
        json.dump(result, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
