"""ctypes binding for the fp64 attention oracle (``oracle.c``).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU path never
imports it, and it never imports the GPU path.

All arrays are float64, C-contiguous, ``[B,H,N,d]`` (statistics ``[B,H,N]``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants a mistake in a copy of oracle.c points this at the copy.
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def compile_c(src: str, out: str) -> None:
    """gcc, fp64, OpenMP, no fast-math and no FMA contraction."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so``."""
    if force or not os.path.exists(_LIB):
        compile_c(_SRC, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_fwd.argtypes = [_dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_double, ctypes.c_int, _dp, _dp]
        lib.oracle_fwd_rows.argtypes = [_dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_int64,
                                        _i64p, _dp, _dp]
        lib.oracle_bwd.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                   _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.oracle_fwd_kv.argtypes = [_dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_double, ctypes.c_int, _dp, _dp]
        lib.oracle_bwd_kv.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                      _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        mask_args = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64]
        lib.oracle_fwd_masked.argtypes = ([_dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_double, ctypes.c_int] + mask_args + [_dp, _dp])
        lib.oracle_bwd_masked.argtypes = ([_dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_double, ctypes.c_int] + mask_args +
                                          [_dp, _dp, _dp, _dp, _dp, _dp, _dp])
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    if a.ndim != 4:
        raise ValueError("expected a [B,H,N,d] array")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


def _block_mask(block_mask, B, H, N, block):
    """(mask array, nb, per-head stride in bytes) for the C side; block_mask is
    [nb, nb] (one mask for every head) or [B, H, nb, nb], nonzero = kept."""
    nb = (N + block - 1) // block
    m = np.ascontiguousarray(block_mask, dtype=np.uint8)
    if m.shape == (nb, nb):
        return m, nb, 0
    if m.shape == (B, H, nb, nb):
        return m, nb, nb * nb
    raise ValueError(f"block mask must be [{nb},{nb}] or [{B},{H},{nb},{nb}], got {m.shape}")


def fwd(q, k, v, scale: float, causal: bool, block_mask=None, block: int = 128):
    """Standard attention forward: returns (O [B,H,N,d], lse [B,H,N]).

    With ``block_mask`` (block-sparse attention), pair (i, j) is kept only if
    ``block_mask[i // block, j // block]`` is nonzero (per head if the mask is
    [B, H, nb, nb]); rows with no kept key get O = 0 and lse = -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape")
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    if block_mask is None:
        _load().oracle_fwd(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale), int(bool(causal)),
                           _ptr(o), _ptr(lse))
    else:
        m, nb, stride = _block_mask(block_mask, B, H, N, block)
        _load().oracle_fwd_masked(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale), int(bool(causal)),
                                  m.ctypes.data, nb, block, stride, _ptr(o), _ptr(lse))
    return o, lse


def fwd_kv(q, k, v, scale: float, causal: bool):
    """Attention of Nq queries ([B,H,Nq,d]) over Nk cached keys and values ([B,H,Nk,d]),
    the queries being the last Nq positions (causal: query t sees keys j <= t + Nk - Nq; with
    Nq > Nk the first Nq - Nk rows see none: O = 0, lse = -inf).
    Returns (O [B,H,Nq,d], lse [B,H,Nq])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B,H,Nk,d] with q's B, H and d")
    o = np.empty_like(q)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    _load().oracle_fwd_kv(_ptr(q), _ptr(k), _ptr(v), B, H, Nq, Nk, d, float(scale), int(bool(causal)),
                          _ptr(o), _ptr(lse))
    return o, lse


def fwd_rows(q, k, v, scale: float, causal: bool, rows):
    """Forward for selected flat rows ``(b*H + h)*N + i``: returns (O_rows [n,d], lse_rows [n])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= B * H * N):
        raise ValueError("row index out of range")
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    _load().oracle_fwd_rows(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale),
                            int(bool(causal)), rows.size,
                            rows.ctypes.data_as(_i64p), _ptr(o), _ptr(lse))
    return o, lse


def bwd(q, k, v, dout, scale: float, causal: bool, block_mask=None, block: int = 128) -> dict:
    """Forward plus analytic backward of ``L = sum(dout * O)``.

    Returns a dict with o, lse, dq, dk, dv, D_pdp (sum_j P_ij dP_ij) and D_odo (dO_i . O_i).
    ``block_mask`` / ``block`` as in :func:`fwd`.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    for t in (k, v, dout):
        if t.shape != q.shape:
            raise ValueError("q, k, v, dout must share one shape")
    out = {name: np.empty_like(q) for name in ("o", "dq", "dk", "dv")}
    for name in ("lse", "D_pdp", "D_odo"):
        out[name] = np.empty((B, H, N), dtype=np.float64)
    outs = [_ptr(out[n]) for n in ("o", "lse", "dq", "dk", "dv", "D_pdp", "D_odo")]
    if block_mask is None:
        _load().oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, d, float(scale),
                           int(bool(causal)), *outs)
    else:
        m, nb, stride = _block_mask(block_mask, B, H, N, block)
        _load().oracle_bwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, d, float(scale),
                                  int(bool(causal)), m.ctypes.data, nb, block, stride, *outs)
    return out


def bwd_kv(q, k, v, dout, scale: float, causal: bool) -> dict:
    """Forward plus analytic backward of ``L = sum(dout * O)`` for Nq queries ([B,H,Nq,d], the
    last positions of the sequence) over Nk keys and values ([B,H,Nk,d]); causal alignment as
    :func:`fwd_kv`. Returns the dict of :func:`bwd` (dq, D_* and lse over Nq rows, dk, dv over Nk)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("k, v must be [B,H,Nk,d] and dout [B,H,Nq,d] with q's B, H and d")
    out = {"o": np.empty_like(q), "dq": np.empty_like(q), "dk": np.empty_like(k), "dv": np.empty_like(k)}
    for name in ("lse", "D_pdp", "D_odo"):
        out[name] = np.empty((B, H, Nq), dtype=np.float64)
    outs = [_ptr(out[n]) for n in ("o", "lse", "dq", "dk", "dv", "D_pdp", "D_odo")]
    _load().oracle_bwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, Nq, Nk, d, float(scale),
                          int(bool(causal)), *outs)
    return out
