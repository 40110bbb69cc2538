"""libfa.so on the host: it loads, exports every function include/fa.h declares,
and rejects every invalid argument before touching the GPU (so these calls run
without one). No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import io_aware_tiled_07_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

A = 0x100000  # fake, 16-byte aligned device addresses: never dereferenced on these paths
GAP = 1 << 30


def ptrs(n):
    return [A + i * GAP for i in range(n)]


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        pytest.skip("libfa.so not built")
    return fa.load()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == {"fa_fwd", "fa_bwd", "fa_bwd_dq", "fa_bwd_prep", "fa_bwd_main",
                          "fa_bwd_workspace_size", "fa_status_string", "fa_fwd_sparse", "fa_bwd_sparse",
                          "fa_fwd_sparse_workspace_size", "fa_bwd_sparse_workspace_size", "fa_fwd_fp8",
                          "fa_decode", "fa_decode_workspace_size", "fa_decode_noalloc", "fa_fwd_general",
                          "fa_bwd_general_workspace_size", "fa_bwd_general"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(6):
        assert fa.fa_status_string(code)
    assert "unknown" in fa.fa_status_string(99)


def test_workspace_size(lib):
    def up(x):
        return (x + 255) // 256 * 256
    rows = 8 * 12 * 1024
    assert fa.fa_bwd_workspace_size(8, 12, 1024, 64, fa.FA_BF16) == 2 * up(rows * 4) + up(rows * 64 * 4)
    assert fa.fa_bwd_workspace_size(1, 1, 7, 64, fa.FA_FP32) == 2 * up(7 * 4)
    assert fa.fa_bwd_workspace_size(0, 1, 7, 64, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 7, 64, 9) == 0


def fwd(lib, q=None, k=None, v=None, o=None, lse=None, B=2, H=3, N=100, d=64, scale=0.125, causal=0, dtype=0):
    p = ptrs(5)
    args = [p[0] if q is None else q, p[1] if k is None else k, p[2] if v is None else v,
            p[3] if o is None else o, p[4] if lse is None else lse]
    return lib.fa_fwd(*[ctypes.c_void_p(x) for x in args], B, H, N, d, ctypes.c_float(scale), causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=0), fa.FA_ERR_INVALID_ARG),
    (dict(v=A + 8), fa.FA_ERR_INVALID_ARG),          # misaligned
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=2, d=128), fa.FA_ERR_UNSUPPORTED),    # fp32 path is d = 64 only
    (dict(o=A), fa.FA_ERR_INVALID_ARG),               # o aliases q
    (dict(lse=A + GAP + 64), fa.FA_ERR_INVALID_ARG),  # lse inside k
    (dict(N=(1 << 27) + 1), fa.FA_ERR_INVALID_ARG),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def bwd(lib, B=2, H=3, N=100, d=64, scale=0.125, causal=0, dtype=0, strategy=0, ws=None, ws_bytes=None, **over):
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"]
    p = dict(zip(names, ptrs(9)))
    p.update({k: v for k, v in over.items() if k in names})
    need = fa.fa_bwd_workspace_size(B, H, N, d, dtype) if dtype in (0, 1, 2) else 0
    ws = A + 9 * GAP if ws is None else ws
    ws_bytes = need if ws_bytes is None else ws_bytes
    return lib.fa_bwd_dq(*[ctypes.c_void_p(p[n]) for n in names], B, H, N, d, ctypes.c_float(scale), causal,
                         dtype, strategy, ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,code", [
    (dict(do=0), fa.FA_ERR_INVALID_ARG),
    (dict(dk=A + 4 * GAP + 2), fa.FA_ERR_INVALID_ARG),
    (dict(d=128, strategy=fa.FA_DQ_ATOMIC), fa.FA_ERR_UNSUPPORTED),  # atomic dQ is d = 64 only
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),             # 16-bit backward: d in {64, 128}
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(strategy=3), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=0), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 9 * GAP + 4), fa.FA_ERR_WORKSPACE),  # misaligned workspace
    (dict(ws=A + 9 * GAP + 128), fa.FA_ERR_WORKSPACE),  # workspace not 256-byte aligned
    (dict(dq=A + 2 * GAP), fa.FA_ERR_INVALID_ARG),    # dq aliases v
    (dict(dv=A + 6 * GAP), fa.FA_ERR_INVALID_ARG),    # dv aliases dq
    (dict(ws=A + 5 * GAP), fa.FA_ERR_INVALID_ARG),    # workspace overlaps lse
    (dict(causal=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
])
def test_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_fa_bwd_is_default_strategy(lib):
    p = [ctypes.c_void_p(x) for x in ptrs(9)]
    st = lib.fa_bwd(*p, 2, 3, 100, 96, ctypes.c_float(0.125), 0, 0, ctypes.c_void_p(A + 9 * GAP),
                    ctypes.c_size_t(1 << 20), None)
    assert st == fa.FA_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib
    monkeypatch.setattr(fa, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        fa.load()
    importlib.reload(fa)


def prep(lib, B=2, H=3, N=100, d=64, dtype=0, strategy=0, o=None, do=None, lse=None, ws=None, ws_bytes=None):
    p = ptrs(3)
    need = fa.fa_bwd_workspace_size(B, H, N, d, dtype) if dtype in (0, 1, 2) else 0
    ws = A + 9 * GAP if ws is None else ws
    ws_bytes = need if ws_bytes is None else ws_bytes
    args = [p[0] if o is None else o, p[1] if do is None else do, p[2] if lse is None else lse]
    return lib.fa_bwd_prep(*[ctypes.c_void_p(x) for x in args], B, H, N, d, dtype, strategy, ctypes.c_void_p(ws),
                           ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,code", [
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=A + 2 * GAP + 4), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=128, strategy=fa.FA_DQ_ATOMIC), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_UNSUPPORTED),
    (dict(strategy=7), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=0), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + GAP), fa.FA_ERR_INVALID_ARG),         # workspace overlaps dout
])
def test_prep_rejects(lib, kw, code):
    assert prep(lib, **kw) == code


def test_prep_fp32_is_a_validated_no_op(lib):
    """For fp32 the first stage only validates (the fp32 backward forms D itself):
    with valid arguments it returns FA_OK without launching anything."""
    assert prep(lib, dtype=fa.FA_FP32) == fa.FA_OK


@pytest.mark.parametrize("strategy", [fa.FA_DQ_DEFAULT, fa.FA_DQ_SEPARATE, fa.FA_DQ_ATOMIC])
@pytest.mark.parametrize("dtype", [fa.FA_BF16, fa.FA_FP16])
@pytest.mark.parametrize("d", [64, 128])
def test_prep_launches_for_16bit(lib, strategy, dtype, d):
    """The 16-bit backward's first stage enqueues its prep kernel for every head
    dim and strategy: on this host (no GPU) the launch fails with FA_ERR_HIP,
    after every argument check has passed. (16-bit d = 128 has no atomic
    strategy.)"""
    want = fa.FA_ERR_UNSUPPORTED if (d == 128 and strategy == fa.FA_DQ_ATOMIC) else fa.FA_ERR_HIP
    assert prep(lib, dtype=dtype, d=d, strategy=strategy) == want


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=128, strategy=fa.FA_DQ_ATOMIC), fa.FA_ERR_UNSUPPORTED),
    (dict(strategy=3), fa.FA_ERR_UNSUPPORTED),
    (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE),
    (dict(dk=A + 6 * GAP), fa.FA_ERR_INVALID_ARG),    # dk aliases dq
])
def test_main_rejects(lib, kw, code):
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"]
    p = dict(zip(names, ptrs(9)))
    p.update({k: v for k, v in kw.items() if k in names})
    d = kw.get("d", 64)
    need = fa.fa_bwd_workspace_size(2, 3, 100, d, 0)
    ws_bytes = kw.get("ws_bytes", need)
    st = lib.fa_bwd_main(*[ctypes.c_void_p(p[n]) for n in names], 2, 3, 100, d, ctypes.c_float(0.125), 0, 0,
                         kw.get("strategy", 0), ctypes.c_void_p(A + 9 * GAP), ctypes.c_size_t(ws_bytes), None)
    assert st == code


def test_library_never_allocates():
    """The library allocates no device or host memory of its own: no allocation or
    free routine of the HIP runtime is among the symbols it imports."""
    import shutil
    import subprocess
    if not os.path.exists(fa.library_path()):
        pytest.skip("libfa.so not built")
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", fa.library_path()], capture_output=True, text=True,
                         check=True).stdout
    imported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert any(s.startswith("hip") for s in imported), "expected HIP runtime imports"
    forbidden = sorted(s for s in imported if re.match(r"hip(Ext)?(Malloc|Free|HostMalloc|HostFree|MallocAsync|"
                                                        r"FreeAsync|MallocManaged|HostAlloc|MemAlloc)", s))
    assert forbidden == []


# ---------------------------------------------------------------- block-sparse entry points

def test_sparse_workspace_sizes(lib):
    def up(x):
        return (x + 255) // 256 * 256
    nb, W = 128, 2  # N = 16384: 128 blocks per side, two 64-bit words per mask row
    assert fa.fa_fwd_sparse_workspace_size(1, 16, 16384, 0) == 2 * up(nb * W * 8)
    assert fa.fa_fwd_sparse_workspace_size(1, 16, 16384, nb * nb) == 2 * up(16 * nb * W * 8)
    rows = 2 * 3 * 1000
    assert fa.fa_bwd_sparse_workspace_size(2, 3, 1000, 0) == 2 * up(rows * 4) + 2 * up(8 * 8)
    assert fa.fa_fwd_sparse_workspace_size(0, 1, 10, 0) == 0
    assert fa.fa_bwd_sparse_workspace_size(1, 1, 10, -1) == 0


def sparse_fwd(lib, B=2, H=3, N=1000, d=64, dtype=0, mask=None, stride=0, ws=None, ws_bytes=None, **over):
    names = ["q", "k", "v", "o", "lse"]
    p = dict(zip(names, ptrs(5)))
    p.update({k: v for k, v in over.items() if k in names})
    mask = A + 6 * GAP if mask is None else mask
    need = fa.fa_fwd_sparse_workspace_size(B, H, N, max(stride, 0))
    ws = A + 7 * GAP if ws is None else ws
    ws_bytes = need if ws_bytes is None else ws_bytes
    return lib.fa_fwd_sparse(*[ctypes.c_void_p(p[n]) for n in names], B, H, N, d, ctypes.c_float(0.125), 0, dtype,
                             ctypes.c_void_p(mask), stride, ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)


def sparse_bwd(lib, B=2, H=3, N=1000, d=64, dtype=0, mask=None, stride=0, ws=None, ws_bytes=None, **over):
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"]
    p = dict(zip(names, ptrs(9)))
    p.update({k: v for k, v in over.items() if k in names})
    mask = A + 10 * GAP if mask is None else mask
    need = fa.fa_bwd_sparse_workspace_size(B, H, N, max(stride, 0))
    ws = A + 11 * GAP if ws is None else ws
    ws_bytes = need if ws_bytes is None else ws_bytes
    return lib.fa_bwd_sparse(*[ctypes.c_void_p(p[n]) for n in names], B, H, N, d, ctypes.c_float(0.125), 0, dtype,
                             ctypes.c_void_p(mask), stride, ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)


SPARSE_REJECTS = [
    (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),   # 16-bit only
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(mask=0), fa.FA_ERR_INVALID_ARG),             # no mask
    (dict(stride=5), fa.FA_ERR_INVALID_ARG),           # per-head masks would overlap (nb * nb = 64)
    (dict(stride=-64), fa.FA_ERR_INVALID_ARG),
    (dict(ws=0), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=64), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 12 * GAP + 64), fa.FA_ERR_WORKSPACE),  # not 256-byte aligned
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,code", SPARSE_REJECTS + [
    (dict(o=A), fa.FA_ERR_INVALID_ARG),                # o aliases q
    (dict(ws=A + 6 * GAP), fa.FA_ERR_INVALID_ARG),     # workspace overlaps the mask
    (dict(o=A + 6 * GAP), fa.FA_ERR_INVALID_ARG),      # o overlaps the mask
])
def test_fwd_sparse_rejects(lib, kw, code):
    assert sparse_fwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", SPARSE_REJECTS + [
    (dict(dk=A), fa.FA_ERR_INVALID_ARG),               # dk aliases q
    (dict(ws=A + 10 * GAP), fa.FA_ERR_INVALID_ARG),    # workspace overlaps the mask
    (dict(dq=A + 10 * GAP), fa.FA_ERR_INVALID_ARG),    # dq overlaps the mask
])
def test_bwd_sparse_rejects(lib, kw, code):
    assert sparse_bwd(lib, **kw) == code


# ---------------------------------------------------------------- FP8 forward

def fwd8(lib, B=2, H=3, N=100, d=64, qd=1.0, kd=1.0, vd=0.5, causal=0, **over):
    names = ["q", "k", "v", "o", "lse"]
    p = dict(zip(names, ptrs(5)))
    p.update({k: v for k, v in over.items() if k in names})
    return lib.fa_fwd_fp8(*[ctypes.c_void_p(p[n]) for n in names], B, H, N, d, ctypes.c_float(0.125), causal,
                          ctypes.c_float(qd), ctypes.c_float(kd), ctypes.c_float(vd), None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(qd=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(kd=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(vd=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=A + 4 * GAP + 4), fa.FA_ERR_INVALID_ARG),   # misaligned
    (dict(o=A + GAP), fa.FA_ERR_INVALID_ARG),             # o aliases k
])
def test_fwd_fp8_rejects(lib, kw, code):
    assert fwd8(lib, **kw) == code


# ---------------------------------------------------------------- attention over a key/value cache

def test_decode_workspace_size(lib):
    # 8 x 32 heads over 16384 keys: about 1,024 workgroups, so 4096 keys per split, 4 splits
    def up(x):
        return (x + 255) // 256 * 256
    rows = 8 * 32 * 4 * 1
    assert fa.fa_decode_workspace_size(8, 32, 1, 16384, 128) == up(rows * 128 * 4) + up(rows * 4)
    # a small cache: one split of at least 256 keys
    assert fa.fa_decode_workspace_size(1, 2, 4, 100, 64) == up(2 * 4 * 64 * 4) + up(2 * 4 * 4)
    assert fa.fa_decode_workspace_size(1, 2, 0, 100, 64) == 0


def dec(lib, B=2, H=3, Nq=1, Nk=1000, d=64, causal=1, dtype=0, ws=None, ws_bytes=None, **over):
    names = ["q", "k", "v", "o", "lse"]
    p = dict(zip(names, ptrs(5)))
    p.update({k: v for k, v in over.items() if k in names})
    need = fa.fa_decode_workspace_size(B, H, max(Nq, 1), max(Nk, 1), d)
    ws = A + 6 * GAP if ws is None else ws
    ws_bytes = need if ws_bytes is None else ws_bytes
    return lib.fa_decode(*[ctypes.c_void_p(p[n]) for n in names], B, H, Nq, Nk, d, ctypes.c_float(0.125), causal,
                         dtype, ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nq=9), fa.FA_ERR_UNSUPPORTED),               # at most 8 queries
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=4, Nk=3), fa.FA_ERR_INVALID_ARG),         # causal needs Nk >= Nq
    (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(k=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=A + GAP), fa.FA_ERR_INVALID_ARG),          # o aliases k
    (dict(ws=0), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=8), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 6 * GAP + 16), fa.FA_ERR_WORKSPACE),  # not 256-byte aligned
    (dict(ws=A + 2 * GAP), fa.FA_ERR_INVALID_ARG),     # workspace overlaps v
])
def test_decode_rejects(lib, kw, code):
    assert dec(lib, **kw) == code


def dec_noalloc(lib, B=2, H=3, Nq=1, Nk=1000, d=64, causal=1, dtype=0, **over):
    names = ["q", "k", "v", "o", "lse"]
    p = dict(zip(names, ptrs(5)))
    p.update({k: v for k, v in over.items() if k in names})
    return lib.fa_decode_noalloc(*[ctypes.c_void_p(p[n]) for n in names], B, H, Nq, Nk, d, ctypes.c_float(0.125),
                                 causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(Nq=9), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=4, Nk=3), fa.FA_ERR_INVALID_ARG),
    (dict(k=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=A + GAP), fa.FA_ERR_INVALID_ARG),          # o aliases k
    # 4096 x 64 heads of 8 queries, d = 128: one split each, 2 M partial rows (> 16 MiB);
    # tensors 2^40 bytes apart so that they do not overlap
    (dict(B=4096, H=64, Nq=8, Nk=256, d=128, **{n: A + i * (1 << 40) for i, n in enumerate("q k v o lse".split())}),
     fa.FA_ERR_SCRATCH),
])
def test_decode_noalloc_rejects(lib, kw, code):
    """Every check, including the scratch limit, runs before any HIP call."""
    assert dec_noalloc(lib, **kw) == code


def test_decode_noalloc_limit_is_the_workspace_size():
    """A shape fits the fixed buffer iff fa_decode's workspace for it does."""
    assert fa.fa_decode_workspace_size(8, 32, 8, 16384, 128) <= fa.FA_DECODE_SCRATCH_BYTES
    assert fa.fa_decode_workspace_size(4096, 64, 8, 256, 128) > fa.FA_DECODE_SCRATCH_BYTES


# ---------------------------------------------------------------- general shapes

def gen(lib, B=2, H=3, Nq=100, Nk=200, d=64, causal=1, dtype=0, st=None, lens=(None, None), **over):
    names = ["q", "k", "v", "o", "lse"]
    p = dict(zip(names, ptrs(5)))
    p.update({k: v for k, v in over.items() if k in names})
    bshd = lambda n: fa._Strides(n * H * d, d, H * d)
    ss = st or [bshd(Nq), bshd(Nk), bshd(Nk), bshd(Nq)]
    return lib.fa_fwd_general(*[ctypes.c_void_p(p[n]) for n in names], B, H, Nq, Nk, d, ctypes.c_float(0.125),
                              causal, dtype, *[ctypes.byref(x) for x in ss],
                              *[ctypes.c_void_p(x) if x else None for x in lens], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(v=A + 2 * GAP + 8), fa.FA_ERR_INVALID_ARG),   # misaligned
    (dict(st=[fa._Strides(0, 64, 4)] * 4), fa.FA_ERR_INVALID_ARG),            # row stride not a multiple of 8
    (dict(st=[fa._Strides(19200, 64, 192), fa._Strides(38400, 64, 192), fa._Strides(38400, 64, 192),
              fa._Strides(19200, 64, 32)]), fa.FA_ERR_INVALID_ARG),         # output rows overlap
    (dict(o=A + GAP), fa.FA_ERR_INVALID_ARG),           # o overlaps k
    (dict(lens=(A + 4 * GAP + 4, None)), fa.FA_ERR_INVALID_ARG),  # lengths overlap lse
])
def test_fwd_general_rejects(lib, kw, code):
    assert gen(lib, **kw) == code


def bgen(lib, B=2, H=3, Nq=100, Nk=200, d=64, causal=1, dtype=0, st=None, lens=(None, None), ws_bytes=None,
         **over):
    names = ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"]
    p = dict(zip(names, ptrs(10)))
    p.update({k: v for k, v in over.items() if k in names})
    bshd = lambda n: fa._Strides(n * H * d, d, H * d)
    rows = [Nq, Nk, Nk, Nq, Nq, Nq, Nk, Nk]  # q k v o dout dq dk dv
    ss = st or [bshd(n) for n in rows]
    need = lib.fa_bwd_general_workspace_size(B, H, Nq)
    return lib.fa_bwd_general(*[ctypes.c_void_p(p[n]) for n in names[:9]], B, H, Nq, Nk, d, ctypes.c_float(0.125),
                              causal, dtype, *[ctypes.byref(x) for x in ss],
                              *[ctypes.c_void_p(x) if x else None for x in lens],
                              ctypes.c_void_p(p["ws"]), need if ws_bytes is None else ws_bytes, None)


def test_bwd_general_workspace_size(lib):
    assert lib.fa_bwd_general_workspace_size(2, 3, 100) == 2 * 2560  # 600 floats, 256-byte rounded, twice
    assert lib.fa_bwd_general_workspace_size(0, 3, 100) == 0
    assert lib.fa_bwd_general_workspace_size(2, 3, 0) == 0


def _bshd_strides(Nq, Nk, H=3, d=64, dk_row=None):
    b = lambda n, r=None: fa._Strides(n * H * d, d, r or H * d)
    return [b(Nq), b(Nk), b(Nk), b(Nq), b(Nq), b(Nq), b(Nk, dk_row), b(Nk)]


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(dq=A + 6 * GAP + 8), fa.FA_ERR_INVALID_ARG),                    # misaligned
    (dict(st=[fa._Strides(0, 64, 4)] * 8), fa.FA_ERR_INVALID_ARG),        # row stride not a multiple of 8
    (dict(st=_bshd_strides(100, 200, dk_row=32)), fa.FA_ERR_INVALID_ARG),  # dk rows overlap each other
    (dict(st=[fa._Strides(0, 1 << 23, 1 << 23)] * 8, B=1, H=1, Nq=1, Nk=1), fa.FA_ERR_INVALID_ARG),  # row stride too large
    (dict(dq=A), fa.FA_ERR_INVALID_ARG),                                   # dq overlaps q
    (dict(dv=A + 7 * GAP), fa.FA_ERR_INVALID_ARG),                         # dv overlaps dk
    (dict(ws=A + 4 * GAP), fa.FA_ERR_INVALID_ARG),                         # workspace overlaps dout
    (dict(lens=(None, A + 8 * GAP + 64)), fa.FA_ERR_INVALID_ARG),          # lengths inside dv
    (dict(ws=0), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=8), fa.FA_ERR_WORKSPACE),
    (dict(ws=A + 9 * GAP + 16), fa.FA_ERR_WORKSPACE),                      # not 256-byte aligned
])
def test_bwd_general_rejects(lib, kw, code):
    assert bgen(lib, **kw) == code
