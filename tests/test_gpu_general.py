"""GPU parity of the forward over general shapes (fa_fwd_general, through the C ABI)
against the fp64 oracle on the same seeded inputs: strided [B,N,H,d] storage,
Nq queries against Nk keys (causal alignment at the end: query i sees keys
j <= i + Nk - Nq; rows that see no key get O = 0, lse = -inf), and sequences of
different lengths padded into one batch. 16-bit tolerance.
"""
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


def bshd(seed, tid, B, N, H, d, dtype="bf16"):
    """A seeded tensor stored [B,N,H,d], returned as its [B,H,N,d] view and the fp64 values in that order."""
    x = seedgen.draw(seed, tid, (B, N, H, d), dtype)
    return x.torch("cuda").transpose(1, 2), np.ascontiguousarray(x.f64.transpose(0, 2, 1, 3))


def check_rows(name, got, ref):
    """Compare rows; rows whose reference lse is -inf must have O = 0 / lse = -inf."""
    check(name, got, ref, "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bshd_layout(causal, d):
    B, N, H = 2, 777, 3
    log(f"general BSHD N={N} causal={causal} d={d}")
    (q, qd), (k, kd), (v, vd) = (bshd(9500 + d, t, B, N, H, d) for t in range(3))
    assert not q.is_contiguous()
    o, lse = fa.fwd_general(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert o.stride() == q.stride()
    o_ref, lse_ref = oracle.fwd(qd, kd, vd, scale_for(d), causal)
    check("o", o, o_ref, "bf16")
    check("lse", lse, lse_ref, "bf16")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(300, 1000), (1, 513), (700, 300)])
def test_queries_against_more_or_fewer_keys(Nq, Nk, causal):
    B, H, d = 2, 2, 64
    log(f"general Nq={Nq} Nk={Nk} causal={causal}")
    q = seedgen.draw(9600 + Nq, 0, (B, H, Nq, d), "bf16")
    k = seedgen.draw(9600 + Nq, 1, (B, H, Nk, d), "bf16")
    v = seedgen.draw(9600 + Nq, 2, (B, H, Nk, d), "bf16")
    o, lse = fa.fwd_general(q.torch("cuda"), k.torch("cuda"), v.torch("cuda"), causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_kv(q.f64, k.f64, v.f64, scale_for(d), causal)
    empty = np.isneginf(lse_ref)
    lg = lse.double().cpu().numpy()
    assert np.array_equal(np.isneginf(lg), empty), "rows without keys must get lse = -inf"
    check("o", o, o_ref, "bf16")
    check("lse", torch.from_numpy(np.where(empty, 0.0, lg)), np.where(empty, 0.0, lse_ref), "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_padded_batch_of_different_lengths(causal):
    """Three sequences padded to 600 rows: per-sequence query and key lengths; rows past a
    sequence's queries are left as they were."""
    B, H, N, d = 3, 2, 600, 64
    lq, lk = [600, 257, 1], [600, 300, 5]
    log(f"general padded batch causal={causal}")
    q, k, v = (seedgen.draw(9700, t, (B, H, N, d), "bf16") for t in range(3))
    o = torch.full((B, H, N, d), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), 7.0, dtype=torch.float32, device="cuda")
    sq = torch.tensor(lq, dtype=torch.int32, device="cuda")
    sk = torch.tensor(lk, dtype=torch.int32, device="cuda")
    fa.fa_fwd_general(q.torch("cuda"), k.torch("cuda"), v.torch("cuda"), o, lse, causal, None, sq, sk)
    torch.cuda.synchronize()
    for b in range(B):
        o_ref, lse_ref = oracle.fwd_kv(q.f64[b:b + 1, :, :lq[b]], k.f64[b:b + 1, :, :lk[b]], v.f64[b:b + 1, :, :lk[b]],
                                       scale_for(d), causal)
        check("o", o[b:b + 1, :, :lq[b]], o_ref, "bf16")
        check("lse", lse[b:b + 1, :, :lq[b]], lse_ref, "bf16")
        assert torch.all(o[b, :, lq[b]:] == 7.0) and torch.all(lse[b, :, lq[b]:] == 7.0)


@pytest.mark.parametrize("causal", [False, True])
def test_contiguous_general_is_the_dense_forward_bitwise(causal):
    q, k, v = (seedgen.draw(9800, t, (2, 3, 1000, 64), "bf16").torch("cuda") for t in range(3))
    o, lse = fa.fwd(q, k, v, causal=causal)
    o2, lse2 = fa.fwd_general(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
