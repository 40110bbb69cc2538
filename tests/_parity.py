"""Helpers for the GPU parity tests: seeded inputs, the oracle side, metrics.

Tolerances (per output tensor): 16-bit inputs need max|diff| <= 2e-2 AND
relRMS = ||diff||_2 / ||ref||_2 <= 1e-2; fp32 inputs need relRMS <= 1e-5.

The max|diff| bar bounds the kernel's own error. An output stored in a 16-bit
type cannot come closer to the fp64 reference than its own rounding, half a
unit in the last place of the reference's binade (bf16: 0.0156 in [4, 8),
0.031 in [8, 16)), so for such outputs each element is held to 2e-2 plus that
half unit; fp32 outputs (lse) are held to 2e-2 exactly.
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


# mantissa bits (without the implicit one) of the 16-bit output types
_MANT = {"torch.bfloat16": 7, "torch.float16": 10}


def half_ulp(ref, mant_bits):
    """Half a unit in the last place of |ref| in a binary type with mant_bits
    stored mantissa bits (normal range; 0 where ref is 0)."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - mant_bits - 1), 0.0)


def check(name, gpu, ref, dtype):
    g = gpu.double().cpu().numpy() if hasattr(gpu, "cpu") else np.asarray(gpu, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    mx, rr = metrics(g, ref)
    log(f"  {name:>4}: max|d|={mx:.3e} relRMS={rr:.3e} max|ref|={np.max(np.abs(ref)):.3f}")
    if dtype == "fp32":
        assert rr <= TOL_32["rel_rms"], f"{name}: relRMS {rr:.3e} > {TOL_32['rel_rms']}"
    else:
        mant = _MANT.get(str(getattr(gpu, "dtype", "")))
        if mant is None or mx <= TOL_16["max_abs"]:
            assert mx <= TOL_16["max_abs"], f"{name}: max|diff| {mx:.3e} > {TOL_16['max_abs']}"
        else:
            # beyond the output's own rounding (module docstring)
            over = np.abs(g - ref) - (TOL_16["max_abs"] + half_ulp(ref, mant))
            worst = float(np.max(over))
            log(f"        max|d| beyond the 16-bit rounding of the output: {mx:.3e} "
                f"(largest excess over 2e-2 + half ulp: {worst:.3e})")
            assert worst <= 0.0, f"{name}: max|diff| {mx:.3e} exceeds 2e-2 + half ulp by {worst:.3e}"
        assert rr <= TOL_16["rel_rms"], f"{name}: relRMS {rr:.3e} > {TOL_16['rel_rms']}"
    return mx, rr


def scale_for(d):
    return 1.0 / math.sqrt(d)
