"""Reentrancy: the C ABI called from several host threads at once, each
thread with its own inputs, outputs, workspace and stream, so the kernels of
different calls run concurrently on the GPU. Every thread's results must equal
(bit for bit: the default kernels are deterministic) what the same calls give
one at a time on the default stream; the sequential results are themselves
checked against the fp64 oracle."""
import math
import threading

import pytest

import io_aware_tiled_07_amd as fa
import oracle
from _parity import check, inputs, log, scale_for

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield


CASES = [  # (seed, (B, H, N, d), causal)
    (9001, (2, 3, 700, 64), True),
    (9002, (1, 4, 1100, 128), False),
    (9003, (3, 2, 513, 64), False),
    (9004, (1, 2, 900, 128), True),
]


def run_case(drawn, shape, causal, stream, reps):
    q, k, v, do = (x.torch("cuda") for x in drawn)
    B, H, N, d = shape
    sc = scale_for(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d, fa.dtype_code(q)), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        fa.fa_fwd(q, k, v, o, lse, causal, sc, stream)
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, causal, sc, ws, stream)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def test_concurrent_calls_from_host_threads_match_sequential():
    drawn = [inputs(seed, shape, "bf16") for seed, shape, _ in CASES]
    ref = []
    for (seed, shape, causal), xs in zip(CASES, drawn):
        log(f"sequential {shape} causal={causal}")
        outs = run_case(xs, shape, causal, torch.cuda.current_stream(), 1)
        r = oracle.bwd(*(x.f64 for x in xs), scale_for(shape[-1]), causal)
        for name, g in zip(("o", "lse", "dq", "dk", "dv"), outs):
            check(name, g, r[name], "bf16")
        ref.append([t.clone() for t in outs])

    results = [None] * len(CASES)
    errors = []

    def worker(i):
        try:
            _, shape, causal = CASES[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                results[i] = run_case(drawn[i], shape, causal, s, 5)
        except Exception as e:  # reported below, in the main thread
            errors.append((i, repr(e)))

    log("concurrent: one host thread and one stream per case, five fwd+bwd each")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i, (outs, want) in enumerate(zip(results, ref)):
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), outs, want):
            assert torch.equal(a, b), f"case {i}: {name} differs from the sequential run"
            assert math.isfinite(float(a.float().abs().max()))
