"""fa_decode_noalloc (the decode entry point that allocates nothing: its split
partials live in the library's fixed per-device scratch buffer) through the C
ABI, against fa_decode with a caller workspace. Both run the same kernels with
the same split plan, so the outputs must agree bit for bit; the first output is
also checked against the fp64 oracle. Two calls in a row, the second on a
smaller input, so the second reads a buffer the first left full."""
import numpy as np
import pytest

import io_aware_tiled_07_amd as fa
import oracle
import seedgen
from _parity import check, log, scale_for

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield


def pair(B, H, Nq, Nk, d, causal, dtype, seed, with_oracle=False):
    log(f"noalloc decode B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} {dtype}")
    draws = [seedgen.draw(seed, t, (B, H, Nq if t == 0 else Nk, d), dtype) for t in range(3)]
    q, k, v = (x.torch("cuda") for x in draws)
    assert fa.fa_decode_workspace_size(B, H, Nq, Nk, d) <= fa.FA_DECODE_SCRATCH_BYTES
    o_ws, lse_ws = fa.decode(q, k, v, causal=causal, scale=scale_for(d))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fa.fa_decode_noalloc(q, k, v, o, lse, causal=causal, scale=scale_for(d))
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws)
    if with_oracle:
        o_ref, lse_ref = oracle.fwd_kv(*(x.f64 for x in draws), scale_for(d), causal)
        check("o", o, o_ref, dtype)
        check("lse", lse, lse_ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_noalloc_decode_matches_workspace_decode(dtype):
    # large first (8 x 32 heads, 4 queries over 16384 keys, d = 128: 4 splits per head),
    # then a smaller call (2 x 4 heads, 1 query over 3000 keys, d = 64)
    pair(8, 32, 4, 16384, 128, True, dtype, 1010, with_oracle=True)
    pair(2, 4, 1, 3000, 64, True, dtype, 1011)
    pair(2, 4, 3, 700, 64, False, dtype, 1012)


def test_noalloc_decode_rejects_oversized_shapes():
    """A shape whose partials exceed the fixed buffer is refused before any launch."""
    B, H, Nq, Nk, d = 4096, 64, 8, 256, 128
    assert fa.fa_decode_workspace_size(B, H, Nq, Nk, d) > fa.FA_DECODE_SCRATCH_BYTES
    lib = fa.load()
    import ctypes
    base = 1 << 44  # never dereferenced: the call returns before any HIP call
    p = [ctypes.c_void_p(base + i * (1 << 40)) for i in range(5)]
    st = lib.fa_decode_noalloc(*p, B, H, Nq, Nk, d, ctypes.c_float(0.1), 1, fa.FA_BF16, None)
    assert st == fa.FA_ERR_SCRATCH
