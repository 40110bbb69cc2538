"""The library's calls captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: the step a training loop would capture (fa_fwd, fa_bwd_prep,
fa_bwd_main with caller-owned workspace) and a decode call through
fa_decode_noalloc. Each is replayed several times with the program's own eager
work and synchronisations between replays, the inputs rewritten in place before
some replays, and every replay compared with an eager run on the same inputs:
the kernels are deterministic, so bit for bit. The first eager result is also
checked against the fp64 oracle."""
import math

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


def draw(seed, shape, dtype, n):
    return [seedgen.draw(seed, t, shape, dtype) for t in range(n)]


@pytest.mark.parametrize("causal", [False, True])
def test_train_step_graph_replays_match_eager(causal):
    B, H, N, d = 2, 4, 640, 64
    log(f"graph step B={B} H={H} N={N} d={d} causal={causal}")
    sc = scale_for(d)
    first = draw(7100 + causal, (B, H, N, d), "bf16", 4)
    second = draw(7200 + causal, (B, H, N, d), "bf16", 4)
    q, k, v, do = (x.torch("cuda") for x in first)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d, fa.dtype_code(q)), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()

    def step():
        fa.fa_fwd(q, k, v, o, lse, causal, sc, s)
        fa.fa_bwd_prep(o, do, lse, ws, fa.FA_DQ_DEFAULT, s)
        fa.fa_bwd_main(q, k, v, o, do, lse, dq, dk, dv, ws, causal, sc, fa.FA_DQ_DEFAULT, s)

    def eager_outputs(src):
        for t, x in zip((q, k, v, do), src):
            t.copy_(x.torch("cuda"))
        with torch.cuda.stream(s):
            step()
        torch.cuda.synchronize()
        return [t.clone() for t in (o, lse, dq, dk, dv)]

    ref1 = eager_outputs(first)
    r = oracle.bwd(*(x.f64 for x in first), sc, causal)
    for name, g in zip(("o", "lse", "dq", "dk", "dv"), ref1):
        check(name, g, r[name], "bf16")
    ref2 = eager_outputs(second)

    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for i, (src, ref) in enumerate([(first, ref1), (first, ref1), (second, ref2), (first, ref1)]):
        for t, x in zip((q, k, v, do), src):
            t.copy_(x.torch("cuda"))
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert math.isfinite(float(junk))
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(a, b), f"replay {i}: {name} differs from the eager run"


def test_noalloc_decode_graph_replays_match_eager():
    B, H, Nq, Nk, d = 4, 8, 4, 3000, 128
    log(f"graph decode B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    sc = scale_for(d)
    first = [seedgen.draw(7300, t, (B, H, Nq if t == 0 else Nk, d), "bf16") for t in range(3)]
    second = [seedgen.draw(7301, t, (B, H, Nq if t == 0 else Nk, d), "bf16") for t in range(3)]
    q, k, v = (x.torch("cuda") for x in first)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()

    def eager_outputs(src):
        for t, x in zip((q, k, v), src):
            t.copy_(x.torch("cuda"))
        with torch.cuda.stream(s):
            fa.fa_decode_noalloc(q, k, v, o, lse, causal=True, scale=sc, stream=s)
        torch.cuda.synchronize()
        return o.clone(), lse.clone()

    ref1 = eager_outputs(first)  # also looks up the scratch buffer before any capture
    o_ref, lse_ref = oracle.fwd_kv(*(x.f64 for x in first), sc, True)
    check("o", ref1[0], o_ref, "bf16")
    check("lse", ref1[1], lse_ref, "bf16")
    ref2 = eager_outputs(second)

    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fa.fa_decode_noalloc(q, k, v, o, lse, causal=True, scale=sc, stream=s)
    torch.cuda.synchronize()
    for i, (src, ref) in enumerate([(first, ref1), (second, ref2), (second, ref2), (first, ref1)]):
        for t, x in zip((q, k, v), src):
            t.copy_(x.torch("cuda"))
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert math.isfinite(float(junk))
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), f"replay {i} differs from the eager run"
