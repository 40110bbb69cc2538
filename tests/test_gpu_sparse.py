"""GPU parity of block-sparse attention: libfa.so's fa_fwd_sparse / fa_bwd_sparse
(through the C ABI) against the fp64 oracle's masked attention on the same
seeded inputs and seeded block masks (128 x 128 blocks).

Reading of the pages (the block-sparse extension is named, not defined): exact
attention with the pairs of every dropped block masked out; a row that keeps no
key has O = 0, lse = -inf and no gradient.
"""
import numpy as np
import pytest

import io_aware_tiled_07_amd as fa
import oracle
import seedgen
from _parity import check, inputs, log, scale_for, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BLOCK = fa.FA_SPARSE_BLOCK


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield


def nblocks(N):
    return (N + BLOCK - 1) // BLOCK


def make_mask(seed, shape, density, diag=True):
    m = seedgen.block_mask(seed, seedgen.TENSOR_MASK, shape, density)
    if diag:  # every query block keeps its own block: no row without keys
        idx = np.arange(shape[-1])
        m[..., idx, idx] = 1
    return m


def run(seed, shape, dtype, causal, mask):
    drawn = inputs(seed, shape, dtype)
    q, k, v, do = to_dev(drawn)
    sc = scale_for(shape[-1])
    m = torch.from_numpy(np.ascontiguousarray(mask)).cuda()
    o, lse = fa.fwd_sparse(q, k, v, m, causal=causal, scale=sc)
    dq, dk, dv = fa.bwd_sparse(q, k, v, o, do, lse, m, causal=causal, scale=sc)
    torch.cuda.synchronize()
    return drawn, (o, lse, dq, dk, dv)


def check_sparse(drawn, outs, dtype, causal, mask, heads=None):
    qd, kd, vd, dod = (x.f64 for x in drawn)
    o, lse, dq, dk, dv = outs
    if heads is not None:
        pick = lambda a: np.stack([a[b, h] for b, h in heads])[None]
        gpick = lambda t: torch.stack([t[b, h] for b, h in heads])[None]
        qd, kd, vd, dod = (pick(a) for a in (qd, kd, vd, dod))
        o, lse, dq, dk, dv = (gpick(t) for t in (o, lse, dq, dk, dv))
        if mask.ndim == 4:
            mask = np.stack([mask[b, h] for b, h in heads])[None]
    r = oracle.bwd(qd, kd, vd, dod, scale_for(qd.shape[-1]), causal, block_mask=mask, block=BLOCK)
    finite = np.isfinite(r["lse"])
    lse_gpu = lse.double().cpu().numpy()
    assert np.array_equal(np.isneginf(lse_gpu), ~finite), "rows without keys must get lse = -inf"
    check("lse", torch.from_numpy(np.where(finite, lse_gpu, 0.0)), np.where(finite, r["lse"], 0.0), dtype)
    for name, g in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        check(name, g, r[name], dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [129, 1000])
def test_sparse_ragged(N, causal, d):
    """Shared seeded mask (density 0.5, diagonal kept), ragged lengths, B*H = 3."""
    log(f"sparse N={N} causal={causal} d={d}")
    mask = make_mask(7000 + N, (nblocks(N), nblocks(N)), 0.5)
    drawn, outs = run(7100 + N + d, (1, 3, N, d), "bf16", causal, mask)
    check_sparse(drawn, outs, "bf16", causal, mask)


@pytest.mark.parametrize("causal", [False, True])
def test_sparse_per_head_masks_with_empty_rows(causal):
    """A mask per head (B*H = 8, the XCD-grouped mapping), density 0.4 with the
    diagonal not forced, so some query blocks keep nothing (O = 0, lse = -inf)."""
    B, H, N, d = 2, 4, 1536, 64
    nb = nblocks(N)
    mask = make_mask(7200, (B, H, nb, nb), 0.4, diag=False)
    mask[0, 0, 3, :] = 0  # at least one query block without keys
    log(f"sparse per-head causal={causal} empty query blocks: {int((mask.sum(-1) == 0).sum())}")
    drawn, outs = run(7300, (B, H, N, d), "bf16", causal, mask)
    check_sparse(drawn, outs, "bf16", causal, mask)
    o, lse, dq = outs[0], outs[1], outs[2]
    assert torch.all(o[0, 0, 384:512] == 0) and torch.all(torch.isneginf(lse[0, 0, 384:512]))
    assert torch.all(dq[0, 0, 384:512] == 0)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp16", 64), ("bf16", 128)])
def test_sparse_long(dtype, d):
    """4096 keys, 2 x 8 heads, shared mask of density 0.25 (diagonal kept), causal:
    two seeded heads checked completely."""
    B, H, N = 2, 8, 4096
    nb = nblocks(N)
    mask = make_mask(7400, (nb, nb), 0.25)
    log(f"sparse long {dtype} d={d} kept blocks {int(mask.sum())}/{nb * nb}")
    drawn, outs = run(7500 + d, (B, H, N, d), dtype, True, mask)
    h0, h1 = (int(x) for x in seedgen.choice_rows(7500, 7, H, 2))
    check_sparse(drawn, outs, dtype, True, mask, heads=[(0, h0), (1, h1)])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_full_mask_is_the_dense_path_bitwise(causal, d):
    """Every block kept: the block-sparse kernels visit the same tiles in the same
    order as the dense ones, so O, lse, dQ, dK, dV agree bit for bit."""
    shape = (2, 4, 1000, d)
    drawn = inputs(7600, shape, "bf16")
    q, k, v, do = to_dev(drawn)
    m = torch.ones((nblocks(1000), nblocks(1000)), dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd(q, k, v, causal=causal)
    o2, lse2 = fa.fwd_sparse(q, k, v, m, causal=causal)
    g = fa.bwd(q, k, v, o, do, lse, causal=causal)
    g2 = fa.bwd_sparse(q, k, v, o, do, lse, m, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip(g, g2):
        assert torch.equal(a, b)


def test_dropped_blocks_are_never_read():
    """NaN in the keys and values of a key block that every query block drops
    reaches nothing (its tiles are never loaded), and its keys get dK = dV = 0."""
    B, H, N, d = 1, 2, 512, 64
    nb = nblocks(N)
    mask = np.ones((nb, nb), dtype=np.uint8)
    mask[:, 2] = 0
    drawn = inputs(7700, (B, H, N, d), "bf16")
    q, k, v, do = to_dev(drawn)
    k[:, :, 256:384] = float("nan")
    v[:, :, 256:384] = float("nan")
    m = torch.from_numpy(mask).cuda()
    o, lse = fa.fwd_sparse(q, k, v, m)
    dq, dk, dv = fa.bwd_sparse(q, k, v, o, do, lse, m)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t).all()
    assert torch.all(dk[:, :, 256:384] == 0) and torch.all(dv[:, :, 256:384] == 0)
    r = oracle.bwd(*(x.f64 for x in drawn), scale_for(d), False, block_mask=mask, block=BLOCK)
    for name, g in (("o", o), ("dq", dq)):
        check(name, g, r[name], "bf16")
