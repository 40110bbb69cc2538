"""Host-side pieces of bench.py (no GPU): FLOP and byte accounting, pinned to the
pages' worked number and to hand arithmetic, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def test_score_grid_of_the_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "score_count.json")))
    assert bench.score_entries(g["tokens"]) == g["score_entries"]


def test_flop_rule():
    w = bench.WORKLOADS["gpt2_small_causal"]
    base = 8 * 12 * 1024 ** 2 * 64
    assert bench.flops(w, "fwd") == 4 * base / 2
    assert bench.flops(w, "step") == 10 * base / 2
    assert bench.flops(bench.WORKLOADS["bert_large"], "fwd") == 4 * 8 * 16 * 512 ** 2 * 64


def test_io_bytes():
    w = bench.WORKLOADS["gpt2_small_causal"]
    fa_b, std_b = bench.io_bytes(w)
    heads, N, d = 8 * 12, 1024, 64
    assert fa_b == heads * (4 * N * d * 2 + 4 * N)         # 50.7 MB
    assert std_b == heads * (4 * N * d + 4 * N * N) * 2    # 856 MB
    assert round(std_b / fa_b, 1) == 16.9


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_algorithmic_bytes_by_hand():
    w = dict(B=1, H=2, N=3, d=4, dtype="bf16")
    t, r = 1 * 2 * 3 * 4 * 2, 1 * 2 * 3 * 4
    assert bench.algorithmic_bytes(w, "fwd") == 4 * t + r          # read Q, K, V; write O, lse
    assert bench.algorithmic_bytes(w, "prep") == 2 * t + 3 * r     # read O, dO, lse; write D, lse2
    assert bench.algorithmic_bytes(w, "main") == 7 * t + 2 * r     # read Q, K, V, dO, lse2, D; write dQ, dK, dV


def test_traffic_is_calibrated_and_goes_stale(monkeypatch):
    monkeypatch.setitem(bench.COUNTERS, "toy", {"main": (100.0, 50.0, 131072.0, 262144.0, "abc")})
    monkeypatch.setattr(bench, "sources_sha", lambda stage: "abc")
    # FETCH_SIZE scaled by 262144 / 131072 = 2, WRITE_SIZE by 1; KiB -> bytes
    assert bench.traffic_bytes("toy", "main") == (200 + 50) * 1024
    monkeypatch.setattr(bench, "sources_sha", lambda stage: "changed")
    assert bench.traffic_bytes("toy", "main") is None
    assert bench.traffic_bytes("toy", "fwd") is None


def test_kept_pairs_by_brute_force():
    """The block-sparse FLOP credit counts exactly the kept (query, key) pairs."""
    import numpy as np
    rng = np.random.default_rng(3)
    for N, causal in ((300, False), (300, True), (129, True), (1, False)):
        nb = (N + 127) // 128
        m = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
        i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
        keep = m[i // 128, j // 128] != 0
        if causal:
            keep &= j <= i
        assert bench.kept_pairs(N, m, causal) == int(keep.sum())
    w = dict(bench.WORKLOADS["gpt2_small_causal"])
    assert bench.pairs_per_head(w) == 1024 * 1024 / 2
    w["pairs"] = 1234
    assert bench.flops(w, "fwd") == 4 * 8 * 12 * 64 * 1234


def test_varlen_lengths_and_pairs():
    """The padded-batch workload's lengths are seeded, inside [N/4, N], and its
    credited pairs are the per-sequence causal rule."""
    w = dict(bench.WORKLOADS["gpt2_varlen_bshd"])
    lens = bench.varlen_lengths(w)
    assert lens.shape == (w["B"],) and lens.min() >= w["N"] // 4 and lens.max() <= w["N"]
    assert (bench.varlen_lengths(w) == lens).all()
    w["pairs"] = float(sum(int(L) ** 2 for L in lens) * 0.5 / w["B"])
    assert bench.flops(w, "step") == 10 * w["H"] * w["d"] * sum(int(L) ** 2 for L in lens) * 0.5


def test_gfx_clock_parse():
    """The clock pass averages the per-XCD GFX clocks of amd-smi's JSON and ignores other clocks."""
    import json

    import bench
    xcd = {f"gfx_{i}": {"clk": {"value": 1900 + 10 * i, "unit": "MHz"}, "max_clk": {"value": 2400, "unit": "MHz"}}
           for i in range(8)}
    xcd["mem_0"] = {"clk": {"value": 2000, "unit": "MHz"}}
    doc = json.dumps({"gpu_data": [{"gpu": 0, "clock": xcd}]})
    assert bench.gfx_clock_mhz(doc) == sum(1900 + 10 * i for i in range(8)) / 8
    assert bench.gfx_clock_mhz(json.dumps({"gpu_data": [{"gpu": 0, "clock": {"mem_0": {"clk": {"value": 1}}}}]})) is None
