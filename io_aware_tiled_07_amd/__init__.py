"""Python binding of libfa.so: exact IO-aware attention on MI355X.

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI (``include/fa.h``). PyTorch provides device memory and
the current stream. There is no fallback: if ``libfa.so`` is missing or a call
fails, an exception is raised.

The raw entry points keep the C names (``fa_fwd``, ``fa_bwd``, ``fa_bwd_dq``,
``fa_bwd_prep``, ``fa_bwd_main``, ``fa_bwd_workspace_size``, ``fa_status_string``,
for block-sparse attention ``fa_fwd_sparse``, ``fa_bwd_sparse`` and their
workspace sizes, the FP8 forward ``fa_fwd_fp8``, and attention over a key/value
cache ``fa_decode`` with ``fa_decode_workspace_size`` (and ``fa_decode_noalloc``, which
uses the library's fixed scratch buffer instead of a workspace), and the forward and
backward over general shapes ``fa_fwd_general``, ``fa_bwd_general``) and take caller-allocated
torch tensors; ``fwd``, ``bwd``, ``fwd_sparse``, ``bwd_sparse``, ``fwd_fp8``,
``decode``, ``fwd_general`` and ``bwd_general`` allocate their outputs.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FA_BF16", "FA_FP16", "FA_FP32", "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED",
    "FA_ERR_WORKSPACE", "FA_ERR_HIP", "FA_DQ_DEFAULT", "FA_DQ_ATOMIC", "FA_DQ_SEPARATE",
    "FaError", "library_path", "load", "fa_status_string", "fa_bwd_workspace_size",
    "fa_fwd", "fa_bwd", "fa_bwd_dq", "fa_bwd_prep", "fa_bwd_main", "fwd", "bwd", "dtype_code",
    "FA_SPARSE_BLOCK", "fa_fwd_sparse_workspace_size", "fa_bwd_sparse_workspace_size", "fa_fwd_sparse",
    "fa_bwd_sparse", "fwd_sparse", "bwd_sparse", "fa_fwd_fp8", "fwd_fp8", "fa_decode_workspace_size",
    "fa_decode", "decode", "fa_decode_noalloc", "FA_ERR_SCRATCH", "FA_DECODE_SCRATCH_BYTES",
    "fa_fwd_general", "fwd_general",
    "fa_bwd_general_workspace_size", "fa_bwd_general", "bwd_general",
]

FA_BF16, FA_FP16, FA_FP32 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_SCRATCH = 0, 1, 2, 3, 4, 5
FA_DECODE_SCRATCH_BYTES = 16 << 20  # fa.h: the fixed scratch buffer of fa_decode_noalloc
FA_DQ_DEFAULT, FA_DQ_ATOMIC, FA_DQ_SEPARATE = 0, 1, 2
FA_SPARSE_BLOCK = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa.so")
_lib = None

_vp, _i, _f, _sz, _ll = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_longlong


class FaError(RuntimeError):
    """A non-zero fa_status from libfa.so."""

    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fa_status_string(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libfa.so (built by ``io_aware_tiled_07_amd.build``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.fa_status_string.argtypes = [_i]
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_bwd_workspace_size.argtypes = [_i, _i, _i, _i, _i]
        lib.fa_bwd_workspace_size.restype = _sz
        lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp]
        lib.fa_fwd.restype = _i
        lib.fa_bwd.argtypes = [_vp] * 9 + [_i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]
        lib.fa_bwd.restype = _i
        lib.fa_bwd_dq.argtypes = [_vp] * 9 + [_i, _i, _i, _i, _f, _i, _i, _i, _vp, _sz, _vp]
        lib.fa_bwd_dq.restype = _i
        lib.fa_bwd_main.argtypes = [_vp] * 9 + [_i, _i, _i, _i, _f, _i, _i, _i, _vp, _sz, _vp]
        lib.fa_bwd_main.restype = _i
        lib.fa_bwd_prep.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]
        lib.fa_bwd_prep.restype = _i
        for name in ("fa_fwd_sparse_workspace_size", "fa_bwd_sparse_workspace_size"):
            getattr(lib, name).argtypes = [_i, _i, _i, _ll]
            getattr(lib, name).restype = _sz
        lib.fa_fwd_sparse.argtypes = [_vp] * 5 + [_i, _i, _i, _i, _f, _i, _i, _vp, _ll, _vp, _sz, _vp]
        lib.fa_fwd_sparse.restype = _i
        lib.fa_bwd_sparse.argtypes = [_vp] * 9 + [_i, _i, _i, _i, _f, _i, _i, _vp, _ll, _vp, _sz, _vp]
        lib.fa_bwd_sparse.restype = _i
        lib.fa_fwd_fp8.argtypes = [_vp] * 5 + [_i, _i, _i, _i, _f, _i, _f, _f, _f, _vp]
        lib.fa_fwd_fp8.restype = _i
        lib.fa_decode_workspace_size.argtypes = [_i, _i, _i, _i, _i]
        lib.fa_decode_workspace_size.restype = _sz
        lib.fa_decode.argtypes = [_vp] * 5 + [_i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]
        lib.fa_decode.restype = _i
        lib.fa_decode_noalloc.argtypes = [_vp] * 5 + [_i, _i, _i, _i, _i, _f, _i, _i, _vp]
        lib.fa_decode_noalloc.restype = _i
        lib.fa_fwd_general.argtypes = [_vp] * 5 + [_i, _i, _i, _i, _i, _f, _i, _i] + [_vp] * 7
        lib.fa_fwd_general.restype = _i
        lib.fa_bwd_general_workspace_size.argtypes = [_i, _i, _i]
        lib.fa_bwd_general_workspace_size.restype = ctypes.c_size_t
        # 9 tensors, 8 scalars, 8 stride structs, 2 length arrays, workspace, bytes, stream
        lib.fa_bwd_general.argtypes = [_vp] * 9 + [_i, _i, _i, _i, _i, _f, _i, _i] + [_vp] * 11 + [ctypes.c_size_t,
                                                                                               _vp]
        lib.fa_bwd_general.restype = _i
        _lib = lib
    return _lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int, dtype: int) -> int:
    return int(load().fa_bwd_workspace_size(B, H, N, d, dtype))


def dtype_code(t) -> int:
    import torch
    codes = {torch.bfloat16: FA_BF16, torch.float16: FA_FP16, torch.float32: FA_FP32}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_bhnd(name, t, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fa_fwd(q, k, v, o, lse, causal: bool = False, scale=None, stream=None) -> None:
    """Enqueue the forward into caller-allocated ``o`` ([B,H,N,d]) and ``lse`` ([B,H,N] float32)."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B,H,N,d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, q.shape, q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    st = load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, N, d, _scale(scale, d), int(bool(causal)), dtype_code(q), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")


def _workspace(q, need, workspace, stream=None):
    """The caller's workspace, or a new one of ``need`` bytes allocated on the
    stream the kernels are enqueued on: the caching allocator then hands the
    block to later work on that stream only, which runs after the kernels, and
    never to work on another stream while they may still use it."""
    import torch
    if workspace is None:
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        with torch.cuda.stream(s):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_bhnd("workspace", workspace)
    return workspace, workspace.numel() * workspace.element_size()


def _bwd_args(q, k, v, o, do, lse, dq, dk, dv, workspace, stream):
    import torch
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bhnd(name, t, q.shape, q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    code = dtype_code(q)
    workspace, nbytes = _workspace(q, fa_bwd_workspace_size(B, H, N, d, code), workspace, stream)
    return code, workspace, nbytes


def fa_bwd_dq(q, k, v, o, do, lse, dq, dk, dv, causal: bool = False, scale=None,
              dq_strategy: int = FA_DQ_DEFAULT, workspace=None, stream=None) -> None:
    """Enqueue the backward into caller-allocated ``dq``, ``dk``, ``dv``. ``workspace`` is a
    device tensor of at least ``fa_bwd_workspace_size`` bytes (allocated here if None)."""
    B, H, N, d = q.shape
    code, workspace, nbytes = _bwd_args(q, k, v, o, do, lse, dq, dk, dv, workspace, stream)
    st = load().fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                          _scale(scale, d), int(bool(causal)), code, int(dq_strategy),
                          workspace.data_ptr(), nbytes, _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dq")


def fa_bwd_prep(o, do, lse, workspace, dq_strategy: int = FA_DQ_DEFAULT, stream=None) -> None:
    """First backward stage: D and lse*log2(e) (and the atomic accumulator's zeroing) into ``workspace``."""
    import torch
    B, H, N, d = o.shape
    _check_bhnd("o", o)
    _check_bhnd("do", do, o.shape, o.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    _check_bhnd("workspace", workspace)
    st = load().fa_bwd_prep(o.data_ptr(), do.data_ptr(), lse.data_ptr(), B, H, N, d, dtype_code(o),
                            int(dq_strategy), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_prep")


def fa_bwd_main(q, k, v, o, do, lse, dq, dk, dv, workspace, causal: bool = False, scale=None,
                dq_strategy: int = FA_DQ_DEFAULT, stream=None) -> None:
    """Second backward stage: dQ, dK, dV from a workspace ``fa_bwd_prep`` filled."""
    B, H, N, d = q.shape
    code, workspace, nbytes = _bwd_args(q, k, v, o, do, lse, dq, dk, dv, workspace, stream)
    st = load().fa_bwd_main(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                            _scale(scale, d), int(bool(causal)), code, int(dq_strategy),
                            workspace.data_ptr(), nbytes, _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_main")


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, causal: bool = False, scale=None, workspace=None,
           stream=None) -> None:
    """``fa_bwd_dq`` with the default dQ strategy."""
    fa_bwd_dq(q, k, v, o, do, lse, dq, dk, dv, causal, scale, FA_DQ_DEFAULT, workspace, stream)


def fwd(q, k, v, causal: bool = False, scale=None, stream=None):
    """Allocate O and lse and run the forward. Returns (o, lse)."""
    import torch
    B, H, N, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, causal, scale, stream)
    return o, lse


def bwd(q, k, v, o, do, lse, causal: bool = False, scale=None, dq_strategy: int = FA_DQ_DEFAULT,
        workspace=None, stream=None):
    """Allocate dQ, dK, dV and run the backward. Returns (dq, dk, dv)."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd_dq(q, k, v, o, do, lse, dq, dk, dv, causal, scale, dq_strategy, workspace, stream)
    return dq, dk, dv


# ---------------------------------------------------------------- block-sparse attention

def fa_fwd_sparse_workspace_size(B: int, H: int, N: int, mask_head_stride: int) -> int:
    return int(load().fa_fwd_sparse_workspace_size(B, H, N, mask_head_stride))


def fa_bwd_sparse_workspace_size(B: int, H: int, N: int, mask_head_stride: int) -> int:
    return int(load().fa_bwd_sparse_workspace_size(B, H, N, mask_head_stride))


def _mask_args(block_mask, B, H, N):
    """(pointer, per-head stride in bytes) of a uint8 device block mask that is
    [nb, nb] (one mask for every head) or [B, H, nb, nb]."""
    import torch
    nb = (N + FA_SPARSE_BLOCK - 1) // FA_SPARSE_BLOCK
    _check_bhnd("block_mask", block_mask, dtype=torch.uint8)
    if tuple(block_mask.shape) == (nb, nb):
        return block_mask.data_ptr(), 0
    if tuple(block_mask.shape) == (B, H, nb, nb):
        return block_mask.data_ptr(), nb * nb
    raise ValueError(f"block_mask must be [{nb},{nb}] or [{B},{H},{nb},{nb}], got {tuple(block_mask.shape)}")


def fa_fwd_sparse(q, k, v, o, lse, block_mask, causal: bool = False, scale=None, workspace=None,
                  stream=None) -> None:
    """Block-sparse forward into caller-allocated ``o`` and ``lse``: 128 x 128 blocks of the
    score matrix whose ``block_mask`` byte is zero are skipped (see ``fa_fwd_sparse`` in fa.h)."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_bhnd(name, t, q.shape, q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    mp, stride = _mask_args(block_mask, B, H, N)
    workspace, nbytes = _workspace(q, fa_fwd_sparse_workspace_size(B, H, N, stride), workspace, stream)
    st = load().fa_fwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              B, H, N, d, _scale(scale, d), int(bool(causal)), dtype_code(q), mp, stride,
                              workspace.data_ptr(), nbytes, _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_sparse")


def fa_bwd_sparse(q, k, v, o, do, lse, dq, dk, dv, block_mask, causal: bool = False, scale=None,
                  workspace=None, stream=None) -> None:
    """Block-sparse backward into caller-allocated ``dq``, ``dk``, ``dv``."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bhnd(name, t, q.shape, q.dtype)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    mp, stride = _mask_args(block_mask, B, H, N)
    workspace, nbytes = _workspace(q, fa_bwd_sparse_workspace_size(B, H, N, stride), workspace, stream)
    st = load().fa_bwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                              lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                              _scale(scale, d), int(bool(causal)), dtype_code(q), mp, stride,
                              workspace.data_ptr(), nbytes, _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_sparse")


def fwd_sparse(q, k, v, block_mask, causal: bool = False, scale=None, stream=None):
    """Allocate O and lse and run the block-sparse forward. Returns (o, lse)."""
    import torch
    B, H, N, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_sparse(q, k, v, o, lse, block_mask, causal, scale, None, stream)
    return o, lse


def bwd_sparse(q, k, v, o, do, lse, block_mask, causal: bool = False, scale=None, stream=None):
    """Allocate dQ, dK, dV and run the block-sparse backward. Returns (dq, dk, dv)."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd_sparse(q, k, v, o, do, lse, dq, dk, dv, block_mask, causal, scale, None, stream)
    return dq, dk, dv


# ---------------------------------------------------------------- FP8 forward

def fa_fwd_fp8(q, k, v, o, lse, causal: bool = False, scale=None, q_descale: float = 1.0,
               k_descale: float = 1.0, v_descale: float = 1.0, stream=None) -> None:
    """FP8 forward into caller-allocated ``o`` ([B,H,N,d] bfloat16) and ``lse``: q, k, v
    hold e4m3 bytes (torch uint8 or float8_e4m3fn), real value = byte value x descale."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B,H,N,d]")
    B, H, N, d = q.shape
    if q.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"q must hold e4m3 bytes, got {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bhnd(name, t, q.shape, q.dtype)
    _check_bhnd("o", o, q.shape, torch.bfloat16)
    _check_bhnd("lse", lse, (B, H, N), torch.float32)
    st = load().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                           _scale(scale, d), int(bool(causal)), float(q_descale), float(k_descale),
                           float(v_descale), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")


def fwd_fp8(q, k, v, causal: bool = False, scale=None, q_descale: float = 1.0, k_descale: float = 1.0,
            v_descale: float = 1.0, stream=None):
    """Allocate O (bfloat16) and lse and run the FP8 forward. Returns (o, lse)."""
    import torch
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q, k, v, o, lse, causal, scale, q_descale, k_descale, v_descale, stream)
    return o, lse


# ---------------------------------------------------------------- attention over a key/value cache

def fa_decode_workspace_size(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(load().fa_decode_workspace_size(B, H, Nq, Nk, d))


def fa_decode(q, k, v, o, lse, causal: bool = True, scale=None, workspace=None, stream=None) -> None:
    """Attention of q ([B,H,Nq,d], the last Nq positions, Nq <= 8) over the cache k, v
    ([B,H,Nk,d]) into caller-allocated ``o`` ([B,H,Nq,d]) and ``lse`` ([B,H,Nq] float32)."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B,H,N,d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check_bhnd("q", q)
    for name, t in (("k", k), ("v", v)):
        _check_bhnd(name, t, (B, H, Nk, d), q.dtype)
    _check_bhnd("o", o, q.shape, q.dtype)
    _check_bhnd("lse", lse, (B, H, Nq), torch.float32)
    workspace, nbytes = _workspace(q, fa_decode_workspace_size(B, H, Nq, Nk, d), workspace, stream)
    st = load().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                          _scale(scale, d), int(bool(causal)), dtype_code(q), workspace.data_ptr(), nbytes,
                          _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_decode")


def fa_decode_noalloc(q, k, v, o, lse, causal: bool = True, scale=None, stream=None) -> None:
    """``fa_decode`` into caller-allocated ``o`` and ``lse`` with the library's fixed
    per-device scratch buffer instead of a workspace: allocates nothing. Calls that may
    overlap on one device share that buffer and must be serialised by the caller."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B,H,N,d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check_bhnd("q", q)
    for name, t in (("k", k), ("v", v)):
        _check_bhnd(name, t, (B, H, Nk, d), q.dtype)
    _check_bhnd("o", o, q.shape, q.dtype)
    _check_bhnd("lse", lse, (B, H, Nq), torch.float32)
    st = load().fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq,
                                  Nk, d, _scale(scale, d), int(bool(causal)), dtype_code(q), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_decode_noalloc")


def decode(q, k, v, causal: bool = True, scale=None, stream=None):
    """Allocate O and lse and run attention over the cache. Returns (o, lse)."""
    import torch
    B, H, Nq, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_decode(q, k, v, o, lse, causal, scale, None, stream)
    return o, lse


# ---------------------------------------------------------------- general shapes

class _Strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong), ("row", ctypes.c_longlong)]


def _strides(t):
    """fa_strides of a [B,H,N,d] torch view whose last dimension is contiguous."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B,H,N,d] view with a contiguous last dimension")
    return _Strides(t.stride(0), t.stride(1), t.stride(2))


def _seqlens(B, seqlens_q, seqlens_k):
    """Device pointers (or None) of the optional per-sequence lengths."""
    import torch
    lens = []
    for name, t in (("seqlens_q", seqlens_q), ("seqlens_k", seqlens_k)):
        if t is None:
            lens.append(None)
        else:
            _check_bhnd(name, t, (B,), torch.int32)
            lens.append(t.data_ptr())
    return lens


def fa_fwd_general(q, k, v, o, lse, causal: bool = False, scale=None, seqlens_q=None, seqlens_k=None,
                   stream=None) -> None:
    """Forward over general shapes: q, o are [B,H,Nq,d] views and k, v [B,H,Nk,d] views with any
    strides (last dimension contiguous), lse [B,H,Nq] float32; seqlens_q / seqlens_k are None or
    int32 device tensors of B lengths (sequences padded into the batch)."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for name, t, n in (("q", q, Nq), ("k", k, Nk), ("v", v, Nk), ("o", o, Nq)):
        if not t.is_cuda or tuple(t.shape) != (B, H, n, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a device tensor [B,H,{n},d] of q's dtype")
    _check_bhnd("lse", lse, (B, H, Nq), torch.float32)
    lens = _seqlens(B, seqlens_q, seqlens_k)
    ss = [_strides(t) for t in (q, k, v, o)]
    st = load().fa_fwd_general(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq,
                               Nk, d, _scale(scale, d), int(bool(causal)), dtype_code(q),
                               *[ctypes.byref(x) for x in ss], lens[0], lens[1], _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_general")


def fwd_general(q, k, v, causal: bool = False, scale=None, seqlens_q=None, seqlens_k=None, stream=None):
    """Allocate O (same layout as q) and lse and run the general-shape forward. Returns (o, lse)."""
    import torch
    B, H, Nq, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_general(q, k, v, o, lse, causal, scale, seqlens_q, seqlens_k, stream)
    return o, lse


def fa_bwd_general_workspace_size(B: int, H: int, Nq: int) -> int:
    return int(load().fa_bwd_general_workspace_size(B, H, Nq))


def fa_bwd_general(q, k, v, o, do, lse, dq, dk, dv, causal: bool = False, scale=None, seqlens_q=None,
                   seqlens_k=None, workspace=None, stream=None) -> None:
    """Backward over general shapes into caller-allocated dq, dk, dv (views of any strides with a
    contiguous last dimension; dq like q, dk / dv like k): the arguments of fa_fwd_general plus o,
    do (dL/dO, like o) and lse as that forward wrote them."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    for name, t, n in (("q", q, Nq), ("k", k, Nk), ("v", v, Nk), ("o", o, Nq), ("do", do, Nq), ("dq", dq, Nq),
                       ("dk", dk, Nk), ("dv", dv, Nk)):
        if not t.is_cuda or tuple(t.shape) != (B, H, n, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a device tensor [B,H,{n},d] of q's dtype")
    _check_bhnd("lse", lse, (B, H, Nq), torch.float32)
    lens = _seqlens(B, seqlens_q, seqlens_k)
    ss = [_strides(t) for t in (q, k, v, o, do, dq, dk, dv)]
    workspace, wbytes = _workspace(q, fa_bwd_general_workspace_size(B, H, Nq), workspace, stream)
    st = load().fa_bwd_general(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Nq, Nk, d,
                               _scale(scale, d), int(bool(causal)), dtype_code(q),
                               *[ctypes.byref(x) for x in ss], lens[0], lens[1], workspace.data_ptr(), wbytes,
                               _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_general")


def bwd_general(q, k, v, o, do, lse, causal: bool = False, scale=None, seqlens_q=None, seqlens_k=None,
                workspace=None, stream=None):
    """Allocate dQ, dK, dV (each in its input's layout) and run the general-shape backward.
    Returns (dq, dk, dv)."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd_general(q, k, v, o, do, lse, dq, dk, dv, causal, scale, seqlens_q, seqlens_k, workspace, stream)
    return dq, dk, dv
