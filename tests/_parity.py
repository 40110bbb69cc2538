"""Helpers for the GPU parity tests: seeded inputs, the oracle side, metrics.

Tolerances (per output tensor): 16-bit inputs need max|diff| <= 2e-2 AND
relRMS = ||diff||_2 / ||ref||_2 <= 1e-2; fp32 inputs need relRMS <= 1e-5.
"""
import math
import sys

import numpy as np

import seedgen

TOL_16 = dict(max_abs=2e-2, rel_rms=1e-2)
TOL_32 = dict(rel_rms=1e-5)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs(seed, shape, dtype, mul=1.0, with_do=True):
    ids = [seedgen.TENSOR_Q, seedgen.TENSOR_K, seedgen.TENSOR_V] + ([seedgen.TENSOR_DO] if with_do else [])
    return [seedgen.draw(seed, t, shape, dtype, mul=mul) for t in ids]


def to_dev(drawn):
    return [d.torch("cuda") for d in drawn]


def metrics(gpu, ref):
    g = gpu.double().cpu().numpy() if hasattr(gpu, "cpu") else np.asarray(gpu, dtype=np.float64)
    diff = g - ref
    denom = np.linalg.norm(ref)
    return float(np.max(np.abs(diff))) if diff.size else 0.0, float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))


def check(name, gpu, ref, dtype):
    g = gpu.double().cpu().numpy() if hasattr(gpu, "cpu") else np.asarray(gpu, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    mx, rr = metrics(g, ref)
    log(f"  {name:>4}: max|d|={mx:.3e} relRMS={rr:.3e} max|ref|={np.max(np.abs(ref)):.3f}")
    if dtype == "fp32":
        assert rr <= TOL_32["rel_rms"], f"{name}: relRMS {rr:.3e} > {TOL_32['rel_rms']}"
    else:
        assert mx <= TOL_16["max_abs"], f"{name}: max|diff| {mx:.3e} > {TOL_16['max_abs']}"
        assert rr <= TOL_16["rel_rms"], f"{name}: relRMS {rr:.3e} > {TOL_16['rel_rms']}"
    return mx, rr


def scale_for(d):
    return 1.0 / math.sqrt(d)
