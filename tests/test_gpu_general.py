"""GPU parity of the forward and backward over general shapes (fa_fwd_general,
fa_bwd_general, through the C ABI) against the fp64 oracle on the same seeded
inputs: strided [B,N,H,d] storage, Nq queries against Nk keys (causal alignment
at the end: query i sees keys j <= i + Nk - Nq; rows that see no key get O = 0,
lse = -inf, dQ = 0), and sequences of different lengths padded into one batch.
16-bit tolerance.
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


# ---------------------------------------------------------------- backward

def check_grads(got, ref, dtype="bf16"):
    for name, g in zip(("dq", "dk", "dv"), got):
        check(name, g, ref[name], dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_bshd_layout(causal, d):
    """[B,N,H,d] storage for every tensor, gradients written in the same layout."""
    B, N, H = 2, 777, 3
    log(f"general bwd BSHD N={N} causal={causal} d={d}")
    (q, qd), (k, kd), (v, vd), (do, dod) = (bshd(9900 + d, t, B, N, H, d) for t in range(4))
    o, lse = fa.fwd_general(q, k, v, causal=causal)
    dq, dk, dv = fa.bwd_general(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    assert dq.stride() == q.stride() and dk.stride() == k.stride()
    check_grads((dq, dk, dv), oracle.bwd(qd, kd, vd, dod, scale_for(d), causal))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,d", [(300, 1000, 64), (1, 513, 64), (700, 300, 64), (200, 650, 128),
                                     (333, 129, 128)])
def test_bwd_queries_against_more_or_fewer_keys(Nq, Nk, d, causal):
    B, H = 2, 2
    log(f"general bwd Nq={Nq} Nk={Nk} d={d} causal={causal}")
    q = seedgen.draw(9910 + Nq, 0, (B, H, Nq, d), "bf16")
    k = seedgen.draw(9910 + Nq, 1, (B, H, Nk, d), "bf16")
    v = seedgen.draw(9910 + Nq, 2, (B, H, Nk, d), "bf16")
    do = seedgen.draw(9910 + Nq, 3, (B, H, Nq, d), "bf16")
    qg, kg, vg, dog = (x.torch("cuda") for x in (q, k, v, do))
    o, lse = fa.fwd_general(qg, kg, vg, causal=causal)
    dq, dk, dv = fa.bwd_general(qg, kg, vg, o, dog, lse, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.bwd_kv(q.f64, k.f64, v.f64, do.f64, scale_for(d), causal)
    check_grads((dq, dk, dv), ref)
    if causal and Nq > Nk:
        assert torch.all(dq[:, :, :Nq - Nk] == 0), "rows without keys must get dQ = 0"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_padded_batch_of_different_lengths(causal, d):
    """Five sequences padded to 600 rows, among them one without queries (its keys get
    dK = dV = 0) and one without keys (its queries get dQ = 0); rows past a sequence's
    queries (dq) or keys (dk, dv) are left as they were."""
    B, H, N = 5, 2, 600
    lq, lk = [600, 257, 1, 0, 30], [600, 300, 5, 40, 0]
    log(f"general bwd padded batch causal={causal} d={d}")
    q, k, v, do = (seedgen.draw(9920 + d, t, (B, H, N, d), "bf16") for t in range(4))
    qg, kg, vg, dog = (x.torch("cuda") for x in (q, k, v, do))
    sq = torch.tensor(lq, dtype=torch.int32, device="cuda")
    sk = torch.tensor(lk, dtype=torch.int32, device="cuda")
    o = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    fa.fa_fwd_general(qg, kg, vg, o, lse, causal, None, sq, sk)
    dq, dk, dv = (torch.full((B, H, N, d), 7.0, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    fa.fa_bwd_general(qg, kg, vg, o, dog, lse, dq, dk, dv, causal, None, sq, sk)
    torch.cuda.synchronize()
    for b in range(B):
        nq, nk = lq[b], lk[b]
        if nq and nk:
            ref = oracle.bwd_kv(q.f64[b:b + 1, :, :nq], k.f64[b:b + 1, :, :nk], v.f64[b:b + 1, :, :nk],
                                do.f64[b:b + 1, :, :nq], scale_for(d), causal)
            check_grads((dq[b:b + 1, :, :nq], dk[b:b + 1, :, :nk], dv[b:b + 1, :, :nk]), ref)
        elif nq:
            assert torch.all(dq[b, :, :nq] == 0)
        elif nk:
            assert torch.all(dk[b, :, :nk] == 0) and torch.all(dv[b, :, :nk] == 0)
        assert torch.all(dq[b, :, nq:] == 7.0), f"sequence {b}: dq rows past its queries were written"
        assert torch.all(dk[b, :, nk:] == 7.0) and torch.all(dv[b, :, nk:] == 7.0), \
            f"sequence {b}: dk / dv rows past its keys were written"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_contiguous_general_bwd_is_the_dense_backward_bitwise(causal, d):
    q, k, v, do = (seedgen.draw(9930 + d, t, (2, 3, 1000, d), "bf16").torch("cuda") for t in range(4))
    o, lse = fa.fwd(q, k, v, causal=causal)
    g1 = fa.bwd(q, k, v, o, do, lse, causal=causal)
    g2 = fa.bwd_general(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
def test_fp16_bshd_queries_against_more_keys(d):
    """fp16, [B,N,H,d] storage, 350 queries against 900 keys, causal: forward and backward."""
    B, H, Nq, Nk = 2, 3, 350, 900
    log(f"general fp16 BSHD Nq={Nq} Nk={Nk} d={d}")
    q = seedgen.draw(9940 + d, 0, (B, Nq, H, d), "fp16")
    k = seedgen.draw(9940 + d, 1, (B, Nk, H, d), "fp16")
    v = seedgen.draw(9940 + d, 2, (B, Nk, H, d), "fp16")
    do = seedgen.draw(9940 + d, 3, (B, Nq, H, d), "fp16")
    qg, kg, vg, dog = (x.torch("cuda").transpose(1, 2) for x in (q, k, v, do))
    o, lse = fa.fwd_general(qg, kg, vg, causal=True)
    dq, dk, dv = fa.bwd_general(qg, kg, vg, o, dog, lse, causal=True)
    torch.cuda.synchronize()
    f = lambda x: np.ascontiguousarray(x.f64.transpose(0, 2, 1, 3))
    ref = oracle.bwd_kv(f(q), f(k), f(v), f(do), scale_for(d), True)
    check("o", o, ref["o"], "fp16")
    check("lse", lse, ref["lse"], "fp16")
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        check(name, g, ref[name], "fp16")
