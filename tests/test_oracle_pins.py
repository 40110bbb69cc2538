"""Pins for the fp64 oracle: each test checks it against something other than
itself (closed forms, invariants, brute force, an independent library, finite
differences), so that a dropped term, a wrong sign or index, or a transposed
operand anywhere in it fails at least one test.

The method's definition (standard attention, same outputs as the naive
formulation) is stated on "FlashAttention: making attention fast by respecting
the memory hierarchy" (paragraphs on the cost of attention and on tiling) and
in the michaelc-yu summary ("What FlashAttention targets"). The backward is
the chain rule through that definition ("Backward / recomputation" names it
only).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from seedgen import normal_f64

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rnd(seed, tid, shape):
    return normal_f64(seed, tid, int(np.prod(shape))).reshape(shape)


def qkv(seed, B, H, N, d):
    return rnd(seed, 0, (B, H, N, d)), rnd(seed, 1, (B, H, N, d)), rnd(seed, 2, (B, H, N, d))


# ---------------------------------------------------------------- probabilities

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    """With d = N and V = identity, O_i is row i of P exactly (one non-zero term per sum)."""
    N = 24
    q, k, _ = qkv(11, 2, 3, N, N)
    v = np.broadcast_to(np.eye(N), (2, 3, N, N)).copy()
    P, _ = oracle.fwd(q * 0.7, k, v, 0.5, causal)
    assert np.all(P >= 0.0)
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-12
    if causal:
        iu = np.triu_indices(N, 1)
        assert np.all(P[..., iu[0], iu[1]] == 0.0), "future keys must get exactly zero weight"
        assert np.all(P[..., np.arange(N), np.arange(N)] > 0.0)


def test_probabilities_brute_force():
    """Each P_ij against a pure-Python softmax of fsum dot products on a tiny head."""
    N, d, scale = 5, 3, 0.8
    q, k, _ = qkv(12, 1, 1, N, d)
    v = np.eye(N).reshape(1, 1, N, N)
    # widen d to N by zero padding q/k columns so V can be the identity
    qp = np.zeros((1, 1, N, N)); qp[..., :d] = q
    kp = np.zeros((1, 1, N, N)); kp[..., :d] = k
    P, lse = oracle.fwd(qp, kp, v, scale, False)
    for i in range(N):
        s = [scale * math.fsum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d)) for j in range(N)]
        z = math.fsum(math.exp(x) for x in s)
        for j in range(N):
            assert abs(P[0, 0, i, j] - math.exp(s[j]) / z) <= 1e-15
        assert abs(lse[0, 0, i] - math.log(z)) <= 1e-14


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_o(causal):
    q, k, _ = qkv(13, 2, 2, 33, 8)
    c = rnd(13, 20, (8,))
    v = np.broadcast_to(c, (2, 2, 33, 8)).copy()
    o, _ = oracle.fwd(q, k, v, 1 / math.sqrt(8), causal)
    assert np.max(np.abs(o - c)) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_uniform_weights(causal):
    """Q = 0 makes every score zero: O_i is the mean of the visible V rows, lse_i = ln(count)."""
    B, H, N, d = 1, 2, 17, 6
    _, k, v = qkv(14, B, H, N, d)
    q = np.zeros_like(k)
    o, lse = oracle.fwd(q, k, v, 0.3, causal)
    for i in range(N):
        n_vis = i + 1 if causal else N
        np.testing.assert_allclose(o[:, :, i], v[:, :, :n_vis].mean(axis=2), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i], math.log(n_vis), rtol=0, atol=1e-14)


def test_single_token():
    """N = 1: softmax over one key is 1, so O = V and lse = scale * q.k."""
    q, k, v = qkv(15, 3, 2, 1, 16)
    o, lse = oracle.fwd(q, k, v, 0.25, False)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.25 * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-14)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_value(x):
    """Fixture numbers are floats or short expressions in ln2 / ln3 / ln4."""
    if isinstance(x, (int, float)):
        return float(x)
    env = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0)}
    return float(eval(x, {"__builtins__": {}}, env))


def test_hand_worked_two_tokens():
    """A 2-token, 1-dim head solved by hand (tests/golden/two_token.json holds the derivation)."""
    g = json.load(open(os.path.join(GOLDEN, "two_token.json")))
    inp = {k: np.array([_golden_value(x) for x in v]).reshape(1, 1, 2, 1)
           for k, v in g["inputs"].items() if k != "scale"}
    for causal, exp in ((False, g["noncausal"]), (True, g["causal"])):
        r = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["dout"], g["inputs"]["scale"], causal)
        for name in ("o", "lse", "dv", "dq", "dk"):
            np.testing.assert_allclose(r[name].ravel(), [_golden_value(x) for x in exp[name]], atol=1e-14,
                                       err_msg=f"{name} causal={causal}")
        if "D" in exp:
            np.testing.assert_allclose(r["D_pdp"].ravel(), [_golden_value(x) for x in exp["D"]], atol=1e-14)


def test_lse_shift():
    """Appending a coordinate with q = 1 and k = c/scale adds c to every score:
    P and O do not change and lse grows by exactly c."""
    B, H, N, d, scale, c = 1, 2, 19, 5, 0.4, 2.75
    q, k, v = qkv(16, B, H, N, d)
    o0, lse0 = oracle.fwd(q, k, v, scale, False)
    q1 = np.concatenate([q, np.ones((B, H, N, 1))], -1)
    k1 = np.concatenate([k, np.full((B, H, N, 1), c / scale)], -1)
    v1 = np.concatenate([v, np.zeros((B, H, N, 1))], -1)
    o1, lse1 = oracle.fwd(q1, k1, v1, scale, False)
    np.testing.assert_allclose(o1[..., :d], o0, atol=1e-13)
    np.testing.assert_allclose(lse1, lse0 + c, atol=1e-13)


# ---------------------------------------------------------------- online softmax equals two-pass

def online_softmax_attention(q, k, v, scale, causal, block):
    """Test-only fp64 online softmax over key blocks of size ``block`` (running max m,
    running sum l, running output rescaled by exp(m_old - m_new)), the reading of the
    tiling paragraph and the "running total" analogy on the groundtruth.day page."""
    B, H, N, d = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                m, l, acc = -np.inf, 0.0, np.zeros(d)
                nk = i + 1 if causal else N
                for j0 in range(0, nk, block):
                    j1 = min(nk, j0 + block)
                    s = scale * (k[b, h, j0:j1] @ q[b, h, i])
                    m_new = max(m, s.max())
                    alpha = math.exp(m - m_new) if m != -np.inf else 0.0
                    p = np.exp(s - m_new)
                    l = alpha * l + p.sum()
                    acc = alpha * acc + p @ v[b, h, j0:j1]
                    m = m_new
                o[b, h, i] = acc / l
                lse[b, h, i] = m + math.log(l)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 7, 64, 200])
def test_online_softmax_matches_two_pass(causal, block):
    q, k, v = qkv(17, 1, 2, 70, 8)
    o_ref, lse_ref = oracle.fwd(q, k, v, 0.35, causal)
    o, lse = online_softmax_attention(q, k, v, 0.35, causal, block)
    tol = 1e-14 if block >= 70 else 1e-13
    assert np.max(np.abs(o - o_ref)) <= tol * max(1.0, np.max(np.abs(o_ref)))
    assert np.max(np.abs(lse - lse_ref)) <= tol * max(1.0, np.max(np.abs(lse_ref)))


# ---------------------------------------------------------------- causal and equivariance

def test_causal_ignores_future():
    """Changing K_j, V_j for every j > i0 leaves rows i <= i0 bitwise unchanged."""
    N, i0 = 40, 17
    q, k, v = qkv(18, 1, 2, N, 8)
    o0, l0 = oracle.fwd(q, k, v, 0.5, True)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i0 + 1:] = rnd(18, 30, k2[:, :, i0 + 1:].shape) * 5
    v2[:, :, i0 + 1:] = rnd(18, 31, v2[:, :, i0 + 1:].shape) * 5
    o1, l1 = oracle.fwd(q, k2, v2, 0.5, True)
    np.testing.assert_array_equal(o1[:, :, :i0 + 1], o0[:, :, :i0 + 1])
    np.testing.assert_array_equal(l1[:, :, :i0 + 1], l0[:, :, :i0 + 1])
    assert np.max(np.abs(o1[:, :, i0 + 1:] - o0[:, :, i0 + 1:])) > 1e-3


def test_permutation_equivariance():
    """Non-causal: permuting K and V rows together changes nothing; permuting Q rows permutes O."""
    N = 23
    q, k, v = qkv(19, 1, 2, N, 6)
    o0, l0 = oracle.fwd(q, k, v, 0.6, False)
    perm = np.argsort(rnd(19, 32, (N,)))
    o1, l1 = oracle.fwd(q, k[:, :, perm], v[:, :, perm], 0.6, False)
    np.testing.assert_allclose(o1, o0, atol=1e-14)
    np.testing.assert_allclose(l1, l0, atol=1e-14)
    o2, l2 = oracle.fwd(q[:, :, perm], k, v, 0.6, False)
    np.testing.assert_array_equal(o2, o0[:, :, perm])
    np.testing.assert_array_equal(l2, l0[:, :, perm])


def test_fwd_rows_matches_fwd():
    q, k, v = qkv(20, 2, 3, 31, 8)
    o, lse = oracle.fwd(q, k, v, 0.5, True)
    rows = np.array([0, 5, 30, 31, 100, 185])
    o_r, lse_r = oracle.fwd_rows(q, k, v, 0.5, True, rows)
    np.testing.assert_array_equal(o_r, o.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(lse_r, lse.reshape(-1)[rows])


# ---------------------------------------------------------------- independent library

@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_cpu_fp64(causal):
    """torch's CPU float64 scaled_dot_product_attention and autograd: an independent implementation."""
    torch = pytest.importorskip("torch")
    B, H, N, d, scale = 2, 3, 29, 16, 0.25
    q, k, v = qkv(21, B, H, N, d)
    do = rnd(21, 3, (B, H, N, d))
    r = oracle.bwd(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(r["o"], to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dq"], tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dk"], tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy(), atol=1e-12)
    s = scale * torch.tensor(q) @ torch.tensor(k).transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(r["lse"], torch.logsumexp(s, -1).numpy(), atol=1e-12)


# ---------------------------------------------------------------- backward

@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    """Central differences of L = sum(dO * O) with step 1e-5 on a tiny problem."""
    B, H, N, d, scale, h = 1, 2, 7, 4, 0.7, 1e-5
    q, k, v = qkv(22, B, H, N, d)
    do = rnd(22, 3, (B, H, N, d))
    r = oracle.bwd(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        return float(np.sum(do * oracle.fwd(q_, k_, v_, scale, causal)[0]))

    for name, x, g in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.linalg.norm(fd - g) / np.linalg.norm(g)
        assert err <= 1e-7, f"d{name}: relative error {err}"


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i; sum_j dV_j = sum_i dO_i (rows of P sum to 1);
    sum_j dK_j = 0 (rows of dS sum to 0)."""
    q, k, v = qkv(23, 2, 2, 37, 8)
    do = rnd(23, 3, q.shape)
    r = oracle.bwd(q, k, v, do, 0.3, causal)
    np.testing.assert_allclose(r["D_pdp"], r["D_odo"], atol=1e-12)
    np.testing.assert_allclose(r["dv"].sum(2), do.sum(2), atol=1e-12)
    np.testing.assert_allclose(r["dk"].sum(2), 0.0, atol=1e-12)
    o, lse = oracle.fwd(q, k, v, 0.3, causal)
    np.testing.assert_array_equal(r["o"], o)
    np.testing.assert_array_equal(r["lse"], lse)


def test_backward_causal_first_key_row():
    """Causal row 0 sees only key 0 (P_00 = 1), so dS_00 = 0 and dQ_0 = 0; the last key is
    seen only by the last row, so dV_{N-1} = P_{N-1,N-1} dO_{N-1} with 0 < P <= 1."""
    q, k, v = qkv(24, 1, 2, 9, 4)
    do = rnd(24, 3, q.shape)
    r = oracle.bwd(q, k, v, do, 0.5, True)
    np.testing.assert_allclose(r["dq"][:, :, 0], 0.0, atol=1e-15)
    ratio = r["dv"][:, :, -1] / do[:, :, -1]
    np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones_like(ratio), rtol=1e-13)
    assert np.all((ratio > 0) & (ratio <= 1))


# ---------------------------------------------------------------- block-sparse attention
# The michaelc-yu summary of Dao et al. names a block-sparse extension of the method
# without defining it. Reading taken: the same attention with more pairs masked; pair
# (i, j) is kept iff the block mask entry [i // block, j // block] is nonzero (and
# j <= i when causal); a row with no kept pair has O = 0, lse = -inf and no gradient.

def element_mask(bm, N, block, causal):
    """[N, N] boolean mask of kept pairs, expanded from a block mask by brute force."""
    keep = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for j in range(N):
            keep[i, j] = bm[i // block, j // block] != 0 and (not causal or j <= i)
    return keep


@pytest.mark.parametrize("causal", [False, True])
def test_full_block_mask_is_dense_attention(causal):
    """Every block kept: exactly the dense oracle, forward and backward, bit for bit."""
    q, k, v = qkv(31, 2, 2, 19, 8)
    do = rnd(31, 3, q.shape)
    nb = 5
    r = oracle.bwd(q, k, v, do, 0.4, causal, block_mask=np.ones((nb, nb)), block=4)
    ref = oracle.bwd(q, k, v, do, 0.4, causal)
    for name in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(r[name], ref[name])


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_mask_is_attention_per_block(causal):
    """Only diagonal blocks kept: each block of rows attends within itself, so the
    result equals dense attention run on each block on its own."""
    block, N = 5, 17
    q, k, v = qkv(32, 1, 2, N, 6)
    do = rnd(32, 3, q.shape)
    nb = (N + block - 1) // block
    r = oracle.bwd(q, k, v, do, 0.6, causal, block_mask=np.eye(nb), block=block)
    for b0 in range(0, N, block):
        sl = slice(b0, min(N, b0 + block))
        ref = oracle.bwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], 0.6, causal)
        for name in ("o", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(r[name][:, :, sl], ref[name], rtol=1e-13, atol=1e-13)


MASK_A = np.array([[1, 0, 1, 0], [1, 1, 0, 0], [0, 1, 1, 1], [1, 0, 0, 1]], dtype=np.uint8)


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_matches_torch_cpu_fp64(causal):
    """torch's CPU float64 attention with the expanded boolean mask, and autograd
    (independent implementation; the mask keeps at least one key in every row)."""
    torch = pytest.importorskip("torch")
    block, N, d, scale = 4, 15, 8, 0.35
    q, k, v = qkv(33, 2, 2, N, d)
    do = rnd(33, 3, q.shape)
    keep = element_mask(MASK_A, N, block, causal)
    assert keep.any(axis=1).all()
    r = oracle.bwd(q, k, v, do, scale, causal, block_mask=MASK_A, block=block)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(keep), scale=scale)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(r["o"], to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dq"], tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dk"], tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy(), atol=1e-12)
    s = scale * torch.tensor(q) @ torch.tensor(k).transpose(-1, -2)
    s = s.masked_fill(~torch.tensor(keep), float("-inf"))
    np.testing.assert_allclose(r["lse"], torch.logsumexp(s, -1).numpy(), atol=1e-12)


def test_block_mask_backward_matches_finite_differences():
    """Central differences of L = sum(dO * O) under a block mask (step 1e-5)."""
    block, N, d, scale, h = 3, 8, 3, 0.8, 1e-5
    bm = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 0]], dtype=np.uint8)
    q, k, v = qkv(34, 1, 1, N, d)
    do = rnd(34, 3, q.shape)
    r = oracle.bwd(q, k, v, do, scale, False, block_mask=bm, block=block)

    def loss(q_, k_, v_):
        return float(np.sum(do * oracle.fwd(q_, k_, v_, scale, False, block_mask=bm, block=block)[0]))

    for name, x, g in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.linalg.norm(fd - g) / np.linalg.norm(g)
        assert err <= 1e-7, f"d{name}: relative error {err}"


def test_masked_out_keys_do_not_matter():
    """Changing keys and values of a dropped block leaves the rows that drop it bitwise
    unchanged, and changes a row that keeps it."""
    block, N = 4, 16
    q, k, v = qkv(35, 1, 1, N, 5)
    o, lse = oracle.fwd(q, k, v, 0.5, False, block_mask=MASK_A, block=block)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 4:8] += 3.0    # key block 1: dropped by query blocks 0 and 2
    v2[:, :, 4:8] -= 2.0
    o2, lse2 = oracle.fwd(q, k2, v2, 0.5, False, block_mask=MASK_A, block=block)
    for qb in range(4):
        rows = slice(4 * qb, 4 * qb + 4)
        if MASK_A[qb, 1]:
            assert np.abs(o2[:, :, rows] - o[:, :, rows]).max() > 1e-3
        else:
            np.testing.assert_array_equal(o2[:, :, rows], o[:, :, rows])
            np.testing.assert_array_equal(lse2[:, :, rows], lse[:, :, rows])


def test_rows_without_keys():
    """A query block whose mask row keeps nothing (or, causal, only later blocks):
    O = 0, lse = -inf, dQ = 0, and its dO does not reach dK or dV."""
    block, N = 4, 12
    bm = np.array([[1, 0, 0], [0, 0, 1], [1, 1, 1]], dtype=np.uint8)  # causal: row block 1 keeps nothing
    q, k, v = qkv(36, 1, 2, N, 4)
    do = rnd(36, 3, q.shape)
    r = oracle.bwd(q, k, v, do, 0.5, True, block_mask=bm, block=block)
    rows = slice(4, 8)
    assert np.all(np.isneginf(r["lse"][:, :, rows]))
    np.testing.assert_array_equal(r["o"][:, :, rows], 0.0)
    np.testing.assert_array_equal(r["dq"][:, :, rows], 0.0)
    do2 = do.copy()
    do2[:, :, rows] = 7.0
    r2 = oracle.bwd(q, k, v, do2, 0.5, True, block_mask=bm, block=block)
    np.testing.assert_array_equal(r2["dk"], r["dk"])
    np.testing.assert_array_equal(r2["dv"], r["dv"])
    assert np.all(np.isfinite(r["lse"][:, :, :4])) and np.all(np.isfinite(r["lse"][:, :, 8:]))


def test_per_head_masks():
    """A [B, H, nb, nb] mask applies head by head: each head equals a run with that
    head's mask shared."""
    block, N = 4, 10
    B, H = 2, 2
    q, k, v = qkv(37, B, H, N, 4)
    nb = 3
    bms = np.stack([np.stack([np.roll(np.eye(nb), s, axis=1) + np.eye(nb) for s in range(b * H, b * H + H)])
                    for b in range(B)]).clip(0, 1)
    o, lse = oracle.fwd(q, k, v, 0.5, False, block_mask=bms, block=block)
    for b in range(B):
        for h in range(H):
            o1, l1 = oracle.fwd(q, k, v, 0.5, False, block_mask=bms[b, h], block=block)
            np.testing.assert_array_equal(o[b, h], o1[b, h])
            np.testing.assert_array_equal(lse[b, h], l1[b, h])


# ---------------------------------------------------------------- queries over a key/value cache
# Decoding with a key/value cache (the pages name the cache beside the method, GT payoff
# paragraph): a few new queries, the last positions of the sequence, attend to every
# cached key (causal: up to their own position).

@pytest.mark.parametrize("causal", [False, True])
def test_cache_with_every_query_is_dense_attention(causal):
    q, k, v = qkv(41, 2, 2, 23, 8)
    o, lse = oracle.fwd_kv(q, k, v, 0.4, causal)
    o2, lse2 = oracle.fwd(q, k, v, 0.4, causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq", [1, 3, 9])
def test_cache_queries_are_the_last_rows(causal, nq):
    """The last nq rows of full attention over the whole sequence, bit for bit."""
    q, k, v = qkv(42, 2, 3, 31, 8)
    o, lse = oracle.fwd_kv(q[:, :, -nq:], k, v, 0.3, causal)
    o2, lse2 = oracle.fwd(q, k, v, 0.3, causal)
    np.testing.assert_array_equal(o, o2[:, :, -nq:])
    np.testing.assert_array_equal(lse, lse2[:, :, -nq:])


def test_cache_matches_torch_cpu_fp64():
    """torch's CPU float64 attention with the bottom-right causal mask (independent)."""
    torch = pytest.importorskip("torch")
    nq, nk, d, scale = 5, 27, 16, 0.25
    q = rnd(43, 0, (2, 2, nq, d))
    k, v = rnd(43, 1, (2, 2, nk, d)), rnd(43, 2, (2, 2, nk, d))
    o, lse = oracle.fwd_kv(q, k, v, scale, True)
    keep = torch.arange(nk)[None, :] <= torch.arange(nq)[:, None] + (nk - nq)
    to = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                                          attn_mask=keep, scale=scale)
    np.testing.assert_allclose(o, to.numpy(), atol=1e-12)
    s = (scale * torch.tensor(q) @ torch.tensor(k).transpose(-1, -2)).masked_fill(~keep, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-12)


def test_cache_with_more_queries_than_keys():
    """Causal with Nq > Nk: the first Nq - Nk queries see no key (O = 0, lse = -inf);
    the others are the rows of a run on the last Nk queries."""
    q = rnd(44, 0, (1, 2, 9, 4))
    k, v = rnd(44, 1, (1, 2, 5, 4)), rnd(44, 2, (1, 2, 5, 4))
    o, lse = oracle.fwd_kv(q, k, v, 0.5, True)
    assert np.all(np.isneginf(lse[:, :, :4]))
    np.testing.assert_array_equal(o[:, :, :4], 0.0)
    o2, lse2 = oracle.fwd_kv(q[:, :, 4:], k, v, 0.5, True)
    np.testing.assert_array_equal(o[:, :, 4:], o2)
    np.testing.assert_array_equal(lse[:, :, 4:], lse2)


# ---------------------------------------------------------------- backward over Nq queries and Nk keys
# The same chain rule over the cache layout: the queries are the last Nq positions, so
# causal masking keeps j <= i + Nk - Nq. Reading taken for general shapes (strided
# layouts, padded batches): each sequence is this computation on its own rows.

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(3, 6), (6, 3)])
def test_backward_kv_matches_finite_differences(causal, nq, nk):
    """Central differences of L = sum(dO * O) through fwd_kv (pinned above), step 1e-5."""
    scale, h = 0.6, 1e-5
    q = rnd(45, 0, (1, 2, nq, 4))
    k, v = rnd(45, 1, (1, 2, nk, 4)), rnd(45, 2, (1, 2, nk, 4))
    do = rnd(45, 3, q.shape)
    r = oracle.bwd_kv(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        o, _ = oracle.fwd_kv(q_, k_, v_, scale, causal)
        return float(np.sum(do * o))

    for name, x, g in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.linalg.norm(fd - g) / max(np.linalg.norm(g), 1e-300)
        assert err <= 1e-7, f"d{name}: relative error {err}"


@pytest.mark.parametrize("causal", [False, True])
def test_backward_kv_is_the_dense_backward_with_silent_rows(causal):
    """Prepend Nk - Nq arbitrary query rows with dO = 0: the dense N = Nk backward
    (pinned by finite differences above) gives the same dK, dV and, on the last
    rows, the same dQ (rows with dO = 0 have dP = 0 and D = 0, so dS = 0)."""
    nq, nk = 5, 13
    qf, k, v = qkv(46, 2, 2, nk, 8)
    do = np.zeros_like(qf)
    do[:, :, -nq:] = rnd(46, 3, (2, 2, nq, 8))
    full = oracle.bwd(qf, k, v, do, 0.45, causal)
    r = oracle.bwd_kv(qf[:, :, -nq:], k, v, do[:, :, -nq:], 0.45, causal)
    np.testing.assert_allclose(r["dq"], full["dq"][:, :, -nq:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["dk"], full["dk"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["dv"], full["dv"], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(r["lse"], full["lse"][:, :, -nq:])


def test_backward_kv_rows_without_keys_and_unseen_keys():
    """Causal, Nq > Nk: the first Nq - Nk queries see no key and get dQ = 0; with Nq < Nk,
    non-causal, every key is seen (dV sums to the sum of dO)."""
    q = rnd(47, 0, (1, 2, 9, 4))
    k, v = rnd(47, 1, (1, 2, 5, 4)), rnd(47, 2, (1, 2, 5, 4))
    do = rnd(47, 3, q.shape)
    r = oracle.bwd_kv(q, k, v, do, 0.5, True)
    np.testing.assert_array_equal(r["dq"][:, :, :4], 0.0)
    r2 = oracle.bwd_kv(q[:, :, 4:], k, v, do[:, :, 4:], 0.5, True)
    for name in ("dk", "dv"):
        np.testing.assert_allclose(r[name], r2[name], rtol=1e-13, atol=1e-14)
    r3 = oracle.bwd_kv(q[:, :, :3], k, v, do[:, :, :3], 0.5, False)
    np.testing.assert_allclose(r3["dv"].sum(2), do[:, :, :3].sum(2), atol=1e-12)
    np.testing.assert_allclose(r3["dk"].sum(2), 0.0, atol=1e-12)
