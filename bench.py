"""Benchmark: exact attention forward + backward through libfa.so on one MI355X.

One step = one pass of the whole path over one batch: fa_fwd (O, lse), then
the backward (fa_bwd_prep: D and lse*log2e; fa_bwd_main: dQ, dK, dV), on the GPT-2-small
shaped causal workload (B=8, H=12, N=1024, d=64, bf16, scale 1/8) unless
--workload says otherwise. Inputs are seeded synthetic Gaussians already
resident in device memory when the timed region starts.

FLOP counting: forward 4*B*H*N^2*d, forward+backward 10*B*H*N^2*d, both halved
for causal. The backward alone is credited with its five matrix products,
10*B*H*N^2*d (halved for causal), whatever the kernels recompute.

The timed region is K whole steps between two HIP events on the stream the
library enqueues on, with nothing else inside it. It comes after the passes
below, which add to the W warm-up steps: the GPU's clock takes several
milliseconds of sustained load to settle (the same 50 GPT-2-small steps timed
right after 10 warm-up steps ran at ~102 us per step against ~85-88 us after the
passes), and the steady state is what a training loop sees. The dominant kernel's
average launch duration (for the roofline entry) comes from a pass of K steps
of its own with events around that kernel's launches only, and the per-stage
breakdown from another pass with events around every launch (each event adds
a little to the step, so neither pass sets the step time). Prints one JSON
line.

``--ceilings`` instead runs the unit microbenchmarks (``fa_ceilings``, built
from ``csrc/ceilings.hip``: chip-wide bf16 MFMA rate and clock, MFMA / FMA /
exp issue mixes per SIMD, LDS read bandwidth per CU, HBM read bandwidth) and
prints their JSON.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA, published
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector, published
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA (published 5.0 PFLOP/s: twice the bf16 rate)
SPARSE_BLOCK = 128         # block size of block-sparse attention (fa.h FA_SPARSE_BLOCK)

WORKLOADS = {
    "gpt2_small_causal": dict(B=8, H=12, N=1024, d=64, causal=True, dtype="bf16", seed=1003, mul=1.0),
    "bert_large": dict(B=8, H=16, N=512, d=64, causal=False, dtype="bf16", seed=1002, mul=1.0),
    "long_causal_16k": dict(B=1, H=16, N=16384, d=64, causal=True, dtype="bf16", seed=1004, mul=1.0),
    # head dim 128 forward + backward (prep pass + fused launch with accumulators in AGPRs)
    "long_causal_8k_d128": dict(B=1, H=16, N=8192, d=128, causal=True, dtype="bf16", seed=1010, mul=1.0),
    # 64K tokens, head dim 128, forward only (inputs scaled by 0.5); the CPU baseline
    # times the oracle on 256 seeded rows, 32 per head
    "wide_64k_fwd": dict(B=1, H=8, N=65536, d=128, causal=False, dtype="bf16", seed=1005, mul=0.5,
                         fwd_only=True, cpu_rows_per_head=32),
    "tiny_fp32": dict(B=1, H=1, N=128, d=64, causal=False, dtype="fp32", seed=1001, mul=1.0),
    # block-sparse attention: one seeded mask of 128 x 128 blocks shared by every head,
    # each block kept with probability 1/4, the diagonal always kept
    "blocksparse_16k": dict(B=1, H=16, N=16384, d=64, causal=False, dtype="bf16", seed=1006, mul=1.0,
                            sparse=dict(density=0.25, mask_seed=1006)),
    # attention of one new query over a 16384-long key/value cache, 8 x 32 heads of 128
    "decode_8x32_16k": dict(B=8, H=32, N=16384, d=128, causal=True, dtype="bf16", seed=1008, mul=1.0,
                            decode=dict(Nq=1)),
    # FP8 (e4m3) forward only, descale factors 1: the long causal shape
    "fp8_fwd_long_causal_16k": dict(B=1, H=16, N=16384, d=64, causal=True, dtype="fp8e4m3", seed=1007, mul=1.0,
                                    fwd_only=True),
    # general shapes: the GPT-2-small causal batch stored [B,N,H,d] ("BSHD"), its eight
    # sequences of seeded lengths uniform over [N/4, N] padded to N rows
    "gpt2_varlen_bshd": dict(B=8, H=12, N=1024, d=64, causal=True, dtype="bf16", seed=1009, mul=1.0,
                             general=dict(len_lo=256)),
}

# kernel names as rocprofv3 reports them, per stage of the default strategy
KERNELS = {"fwd": "fwd_kernel", "prep": "bwd_prep_kernel", "main": "bwd_fused_kernel"}
# source files each stage's kernel is built from (a change to any of them makes
# recorded hardware counters stale)
KERNEL_SOURCES = {"fwd": ("fa_fwd.hip", "fa_device.h"), "prep": ("fa_bwd.hip", "fa_device.h"),
                  "main": ("fa_bwd.hip", "fa_device.h")}

# Beyond-L2 traffic per launch from rocprofv3 --pmc (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch, in runs of their own), for the default dQ strategy, with the
# sha256 (first 16 hex digits) of the kernel's sources when they were taken.
# Each counter is scaled by what it reads for a plain 256 MiB device-to-device
# copy in the same runs (the runtime's copy kernel: FETCH_SIZE 131,089 KiB and
# WRITE_SIZE 262,144 KiB for 262,144 KiB each way). The summaries and the
# commands are in profiles/.
COPY_PROBE_KIB = 262144
COUNTERS = {
    # workload: {stage: (FETCH_SIZE KiB, WRITE_SIZE KiB, copy FETCH_SIZE KiB, copy WRITE_SIZE KiB, sources sha)}
    "gpt2_small_causal": {
        "fwd": (18539.3, 12672.0, 131088.5, 262144.0, "67a35d39f0ef5702"),
        "prep": (12492.7, 768.0, 131088.5, 262144.0, "772f7ee8ed4a0449"),
        "main": (63376.6, 36864.0, 131088.5, 262144.0, "772f7ee8ed4a0449"),
    },
}


def sources_sha(stage):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, "io_aware_tiled_07_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes(workload, stage):
    """Counter-derived bytes per launch, or None when none were recorded for this
    kernel or its sources changed since."""
    rec = COUNTERS.get(workload, {}).get(stage)
    if rec is None or rec[4] != sources_sha(stage):
        return None
    fetch, write, copy_fetch, copy_write, _ = rec
    return round((fetch * COPY_PROBE_KIB / copy_fetch + write * COPY_PROBE_KIB / copy_write) * 1024)


def algorithmic_bytes(w, stage):
    """Bytes a launch must move at least: every input read once, every output written once.
    prep reads o, dout and lse and writes D and lse*log2e; the fused backward reads q, k, v,
    dout, D and lse*log2e and writes dq, dk and dv."""
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    elt = 4 if w["dtype"] == "fp32" else 2
    t, r = B * H * N * d * elt, B * H * N * 4
    return {"fwd": 3 * t + t + r, "prep": 2 * t + r + 2 * r, "main": 4 * t + 2 * r + 3 * t}[stage]


def block_mask(w):
    """The workload's seeded block mask ([nb, nb] uint8, shared by every head), or None."""
    sp = w.get("sparse")
    if sp is None:
        return None
    import numpy as np
    import seedgen
    nb = (w["N"] + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    m = seedgen.block_mask(sp["mask_seed"], seedgen.TENSOR_MASK, (nb, nb), sp["density"])
    m[np.arange(nb), np.arange(nb)] = 1
    return m


def kept_pairs(N, mask, causal):
    """Query-key pairs one head keeps under a block mask (exact count)."""
    import numpy as np
    nb = mask.shape[0]
    total = 0
    for bi in range(nb):
        r0, r1 = bi * SPARSE_BLOCK, min(N, (bi + 1) * SPARSE_BLOCK)
        for bj in np.nonzero(mask[bi])[0].tolist():
            c0, c1 = bj * SPARSE_BLOCK, min(N, (bj + 1) * SPARSE_BLOCK)
            if not causal:
                total += (r1 - r0) * (c1 - c0)
            else:
                i = np.arange(r0, r1)
                total += int(np.clip(np.minimum(c1, i + 1) - c0, 0, None).sum())
    return total


def pairs_per_head(w):
    """Score pairs credited per head: N^2 (halved for causal), or the kept pairs of a block mask."""
    return w["pairs"] if "pairs" in w else w["N"] ** 2 * (0.5 if w["causal"] else 1.0)


def flops(w, which):
    base = w["B"] * w["H"] * w["d"] * pairs_per_head(w)
    mult = {"fwd": 4, "bwd": 10, "step": 10, "step_alg": 14}[which]
    return mult * base


def score_entries(N):
    """Entries of one head's N x N score grid (what standard attention writes out)."""
    return N * N


def io_bytes(w):
    """Forward HBM bytes per launch: FlashAttention's compulsory traffic (read Q, K, V,
    write O and lse) and standard attention's (the same, plus writing the N x N scores,
    reading them for the softmax, writing the probabilities and reading them for PV),
    both at the workload's element size, scores and probabilities at that size too."""
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    elt = {"fp32": 4, "fp8e4m3": 1}.get(w["dtype"], 2)
    out_elt = 2 if w["dtype"] == "fp8e4m3" else elt  # the fp8 forward writes O in bf16
    fa_b = B * H * (3 * N * d * elt + N * d * out_elt + 4 * N)
    std_b = B * H * (4 * N * d + 4 * score_entries(N)) * elt
    return fa_b, std_b


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, shape, scale, causal, min_seconds=10.0):
    """The fp64 oracle (as it stands) on the host cores: whole fwd+bwd passes (forward
    passes for a forward-only workload) over the same seeded inputs, repeated until at
    least ``min_seconds`` have elapsed, or over a subset of (batch, head) pairs when one
    pass would take longer than that."""
    import oracle
    import seedgen
    B, H, N, d = shape
    heads = B * H
    if w.get("cpu_rows_per_head"):
        return cpu_baseline_rows(w, shape, scale, causal, min_seconds)
    drawn = [seedgen.draw(w["seed"], t, shape, w["dtype"], mul=w["mul"]).f64.reshape(heads, N, d) for t in range(4)]
    mask = block_mask(w)
    fwd_only = w.get("fwd_only", False)

    def one_pass(xs):
        if fwd_only:
            oracle.fwd(*xs[:3], scale, causal)
        else:
            oracle.bwd(*xs, scale, causal, block_mask=mask, block=SPARSE_BLOCK)

    # time one head first to size the sample
    one = [x[:1].reshape(1, 1, N, d) for x in drawn]
    t0 = time.perf_counter()
    one_pass(one)
    t_head = max(time.perf_counter() - t0, 1e-6)
    nh = max(1, min(heads, int(min_seconds / t_head)))
    sample = [x[:nh].reshape(1, nh, N, d) for x in drawn]
    reps, t_total = 0, 0.0
    while t_total < min_seconds and reps < 1000:
        t0 = time.perf_counter()
        one_pass(sample)
        t_total += time.perf_counter() - t0
        reps += 1
    credited = flops(dict(w, B=1, H=nh), "fwd" if fwd_only else "step") * reps
    kind = "forward" if fwd_only else "fwd+bwd"
    return {"value": round(credited / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{reps} {kind} pass(es) of the fp64 oracle over {nh} of {heads} (batch, head) pairs "
                      f"of the same workload, {t_total:.2f} s; credited with the same rule as the GPU"}


def cpu_baseline_rows(w, shape, scale, causal, min_seconds=10.0):
    """The fp64 oracle's forward on a seeded sample of query rows (``cpu_rows_per_head`` per
    (batch, head)), for a workload whose single head would take the oracle longer than
    ``min_seconds``; repeated until that much time has elapsed. Credited 4*d per visible
    (query, key) pair, as the GPU."""
    import oracle
    import seedgen
    B, H, N, d = shape
    per = w["cpu_rows_per_head"]
    q, k, v = (seedgen.draw(w["seed"], t, shape, w["dtype"], mul=w["mul"]).f64 for t in range(3))
    rows = np.concatenate([bh * N + seedgen.choice_rows(w["seed"], 16 + bh, N, per) for bh in range(B * H)])
    visible = int(((rows % N) + 1).sum()) if causal else rows.size * N
    reps, t_total = 0, 0.0
    while t_total < min_seconds and reps < 1000:
        t0 = time.perf_counter()
        oracle.fwd_rows(q, k, v, scale, causal, rows)
        t_total += time.perf_counter() - t0
        reps += 1
    credited = 4 * d * visible * reps
    return {"value": round(credited / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{reps} forward pass(es) of the fp64 oracle over {rows.size} seeded query rows "
                      f"({per} per (batch, head)) of the same workload, each against all its keys, "
                      f"{t_total:.2f} s; credited 4*d per visible query-key pair"}


PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published


def gfx_clock_mhz(amd_smi_json):
    """Mean GFX clock (MHz) over the XCDs in the output of `amd-smi metric -g 0 --clock --json`
    (entries gfx_0, gfx_1, ... of gpu_data[0].clock); None if it lists none."""
    clk = json.loads(amd_smi_json)["gpu_data"][0]["clock"]
    vals = [v["clk"]["value"] for key, v in clk.items()
            if key.startswith("gfx_") and isinstance(v.get("clk", {}).get("value"), (int, float))]
    return sum(vals) / len(vals) if vals else None


def sclk_during(run_steps, seconds=3.0):
    """Shader clock while the workload runs: `amd-smi metric --clock` is polled from
    a thread while run_steps() is called back to back for `seconds`; each sample is
    the mean GFX clock over the XCDs it lists (MHz). If no busy sample came back (tool
    missing, unexpected output), mean_mhz is None and "error" says why."""
    import subprocess
    import threading

    import torch
    samples, err = [], []
    stop = threading.Event()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True,
                                   text=True, timeout=20)
                mhz = gfx_clock_mhz(r.stdout)
                if mhz is not None:
                    samples.append(mhz)
            except Exception as e:  # tool missing or output not as expected: report none
                err.append(f"{type(e).__name__}: {e}"[:200])
                return

    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        run_steps()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    # samples below the 500 MHz floor amd-smi lists as min_clk are idle (deep sleep) moments
    busy = [x for x in samples if x >= 500.0]
    if not busy:
        return {"mean_mhz": None, "samples": 0, "idle_samples": len(samples), "error": err[0] if err else "no sample"}
    return {"mean_mhz": round(statistics.mean(busy), 1), "min_mhz": round(min(busy), 1),
            "max_mhz": round(max(busy), 1), "samples": len(busy), "idle_samples": len(samples) - len(busy),
            "source": (f"amd-smi metric --clock, mean over the XCDs, polled while steps ran back to back for "
                       f"{seconds:.0f} s; samples below 500 MHz (idle) left out")}


def decode_bytes(w):
    """Compulsory HBM bytes of one call of attention over the cache: read Q, K, V,
    write O and lse."""
    B, H, Nk, d, Nq = w["B"], w["H"], w["N"], w["d"], w["decode"]["Nq"]
    return B * H * (2 * Nq * d * 2 + 2 * Nk * d * 2 + 4 * Nq)


def run_decode(args, w):
    """Bench line for attention over a key/value cache: HBM bound, so the value is
    compulsory bytes per second."""
    import torch

    import io_aware_tiled_07_amd as fa
    import seedgen
    B, H, Nk, d, Nq = w["B"], w["H"], w["N"], w["d"], w["decode"]["Nq"]
    causal, scale, dev = w["causal"], 1.0 / math.sqrt(d), "cuda"
    q = seedgen.draw(w["seed"], 0, (B, H, Nq, d), w["dtype"], want_f64=False).torch(dev)
    k = seedgen.draw(w["seed"], 1, (B, H, Nk, d), w["dtype"], want_f64=False).torch(dev)
    v = seedgen.draw(w["seed"], 2, (B, H, Nk, d), w["dtype"], want_f64=False).torch(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_decode_workspace_size(B, H, Nq, Nk, d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        fa.fa_decode(q, k, v, o, lse, causal, scale, ws, stream)
    torch.cuda.synchronize()
    K = args.steps
    # per-call durations from a pass of their own (events around every call)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        evs[i][0].record(stream)
        fa.fa_decode(q, k, v, o, lse, causal, scale, ws, stream)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = statistics.mean(a.elapsed_time(b) for a, b in evs)
    # timed region: K calls between two events
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(K):
        fa.fa_decode(q, k, v, o, lse, causal, scale, ws, stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / K
    nbytes = decode_bytes(w)
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    call_gbs = nbytes / (call_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        qd = seedgen.draw(w["seed"], 0, (B, H, Nq, d), w["dtype"]).f64.reshape(B * H, Nq, d)
        kd = seedgen.draw(w["seed"], 1, (B, H, Nk, d), w["dtype"]).f64.reshape(B * H, Nk, d)
        vd = seedgen.draw(w["seed"], 2, (B, H, Nk, d), w["dtype"]).f64.reshape(B * H, Nk, d)
        reps, t_total, nh = 0, 0.0, B * H
        while t_total < 10.0 and reps < 1000:
            a = time.perf_counter()
            oracle.fwd_kv(qd[None, :nh], kd[None, :nh], vd[None, :nh], scale, causal)
            t_total += time.perf_counter() - a
            reps += 1
        cpu = {"value": round(nbytes * reps / t_total / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"{reps} pass(es) of the fp64 oracle over all {nh} heads of the same workload, "
                         f"{t_total:.2f} s; credited with the same compulsory bytes"}
    out = {
        "metric": "attention over a key/value cache: GB/s of compulsory HBM traffic (read Q, K, V; write O, lse)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w["dtype"], "data": "synthetic: seeded i.i.d. N(0,1) query and cache of the workload's shape",
        "config": {"workload": args.workload, "B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d, "causal": causal,
                   "dtype": w["dtype"], "scale": scale},
        "roofline": {"bound": "hbm", "achieved": round(call_gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(call_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes": nbytes, "kernel": "fa_decode: decode_split_kernel + decode_merge_kernel",
                     "avg_launch_ms": round(call_ms, 5)},
        "cpu_baseline": cpu, "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


def varlen_lengths(w):
    """The workload's seeded per-sequence lengths (queries = keys = L_b)."""
    import seedgen
    return seedgen.lengths(w["seed"], seedgen.TENSOR_LENS, w["B"], w["general"]["len_lo"], w["N"])


def run_general(args, w):
    """Bench line for general shapes: fa_fwd_general + fa_bwd_general over a padded
    batch in [B,N,H,d] storage. Credited FLOP: 10*H*d per visible query-key pair of
    each sequence, L_b^2 / 2 per head for causal (the dense rule applied per sequence)."""
    import torch

    import io_aware_tiled_07_amd as fa
    import seedgen
    B, H, N, d, causal = w["B"], w["H"], w["N"], w["d"], w["causal"]
    scale, dev = 1.0 / math.sqrt(d), "cuda"
    lens = varlen_lengths(w)
    pair_rule = 0.5 if causal else 1.0
    w["pairs"] = float(sum(int(L) ** 2 for L in lens) * pair_rule / B)  # mean per head, for flops()
    store = (B, N, H, d)
    q, k, v, do = (seedgen.draw(w["seed"], t, store, w["dtype"], want_f64=False).torch(dev).transpose(1, 2)
                   for t in range(4))
    o, dq, dk, dv = (torch.empty(store, dtype=q.dtype, device=dev).transpose(1, 2) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    sl = torch.from_numpy(lens).to(dev)
    ws = torch.empty(fa.fa_bwd_general_workspace_size(B, H, N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    stages = ("fwd", "main")

    def run(evs=None):
        evs = evs or {}
        for name in stages:
            if name in evs: evs[name][0].record(stream)
            if name == "fwd":
                fa.fa_fwd_general(q, k, v, o, lse, causal, scale, sl, sl, stream)
            else:
                fa.fa_bwd_general(q, k, v, o, do, lse, dq, dk, dv, causal, scale, sl, sl, ws, stream)
            if name in evs: evs[name][1].record(stream)

    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    K = args.steps
    brk = [{name: ev_pair() for name in stages} for _ in range(K)]
    for i in range(K):
        run(brk[i])
    torch.cuda.synchronize()
    stage_ms = {name: statistics.mean(e[name][0].elapsed_time(e[name][1]) for e in brk) for name in stages}
    dom_ev = [{"main": ev_pair()} for _ in range(K)]
    for i in range(K):
        run(dom_ev[i])
    torch.cuda.synchronize()
    dom_ms = statistics.mean(e["main"][0].elapsed_time(e["main"][1]) for e in dom_ev)
    t_start, t_end = ev_pair()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        run()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / K
    tf_step = flops(w, "step") / (ms_step * 1e-3) / 1e12
    dom_tf = flops(w, "bwd") / (dom_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        full = [seedgen.draw(w["seed"], t, store, w["dtype"]).f64.transpose(0, 2, 1, 3) for t in range(4)]
        reps, t_total, credited, b = 0, 0.0, 0.0, 0
        while t_total < 10.0 and reps < 1000:
            L = int(lens[b % B])
            xs = [np.ascontiguousarray(x[b % B:b % B + 1, :, :L]) for x in full]
            a = time.perf_counter()
            oracle.bwd_kv(*xs, scale, causal)
            t_total += time.perf_counter() - a
            credited += 10 * H * d * L * L * pair_rule
            reps += 1
            b += 1
        cpu = {"value": round(credited / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"fwd+bwd of the fp64 oracle over {reps} sequence(s) of the same batch (all heads each), "
                         f"{t_total:.2f} s; credited with the same rule as the GPU"}
    out = {
        "metric": "attention TFLOP/s fwd+bwd over a padded batch (10*H*d per visible pair, L_b^2/2 per head causal)",
        "value": round(tf_step, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic: seeded i.i.d. N(0,1) inputs stored [B,N,H,d], seeded lengths uniform over [N/4, N]",
        "config": {"workload": args.workload, "B": B, "H": H, "N": N, "d": d, "causal": causal, "dtype": w["dtype"],
                   "scale": scale, "layout": "BSHD", "lengths": lens.tolist()},
        "fwd": {"ms": round(stage_ms["fwd"], 5),
                "tflops": round(flops(w, "fwd") / (stage_ms["fwd"] * 1e-3) / 1e12, 3)},
        "bwd": {"ms": round(stage_ms["main"], 5),
                "tflops_10x": round(flops(w, "bwd") / (stage_ms["main"] * 1e-3) / 1e12, 3)},
        "roofline": {"bound": "mfma", "achieved": round(dom_tf, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(dom_tf / peak, 4), "traffic": None, "algorithmic_bytes": None,
                     "kernel": "fa_bwd_general: bwd_prep_kernel (general) + "
                               + ("bwd128_fused_kernel" if d == 128 else "bwd_fused_kernel") + " (general)",
                     "flop_per_launch": flops(w, "bwd"), "avg_launch_ms": round(dom_ms, 5),
                     "flop_rule": "bwd 10*H*d per visible query-key pair of each sequence"},
        "cpu_baseline": cpu, "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt2_small_causal", choices=sorted(WORKLOADS))
    ap.add_argument("--dq", default="default", choices=["default", "atomic", "separate"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip the 3 s pass that samples the shader clock with amd-smi (use under a profiler)")
    ap.add_argument("--flush-mall", action="store_true",
                    help="also time K cold steps, each after writing a 512 MiB scratch buffer (evicts L2 and the "
                         "256 MB Infinity Cache)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters under a profiler)")
    ap.add_argument("--ceilings", action="store_true",
                    help="run the unit microbenchmarks (fa_ceilings) instead of a workload and print their JSON")
    args = ap.parse_args()
    if args.ceilings:
        import subprocess
        exe = os.path.join(ROOT, "io_aware_tiled_07_amd", "fa_ceilings")
        if not os.path.exists(exe):
            raise RuntimeError(f"{exe} is not built; run __graft_entry__.build() first")
        r = subprocess.run([exe], capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stderr)
            sys.exit(r.returncode)
        print(json.dumps({"ceilings": json.loads(r.stdout)}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the kernels are measured on "
              "one GPU's share of the work at its real shape; see the sharding notes in the design document.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import io_aware_tiled_07_amd as fa
    import seedgen

    w = dict(WORKLOADS[args.workload])
    if "decode" in w:
        run_decode(args, w)
        return
    if "general" in w:
        run_general(args, w)
        return
    mask_np = block_mask(w)
    sparse = mask_np is not None
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    if sparse:
        w["pairs"] = kept_pairs(N, mask_np, w["causal"])
    shape = (B, H, N, d)
    scale = 1.0 / math.sqrt(d)
    causal = w["causal"]
    dev = "cuda"
    drawn = [seedgen.draw(w["seed"], t, shape, w["dtype"], mul=w["mul"], want_f64=False) for t in range(4)]
    q, k, v, do = (x.torch(dev) for x in drawn)
    fp8 = w["dtype"] == "fp8e4m3"
    fwd_only = w.get("fwd_only", False)
    o = torch.empty(shape, dtype=torch.bfloat16, device=dev) if fp8 else torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if not fwd_only:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        code = fa.dtype_code(q)
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d, code), dtype=torch.uint8, device=dev)
    strategy = {"default": fa.FA_DQ_DEFAULT, "atomic": fa.FA_DQ_ATOMIC, "separate": fa.FA_DQ_SEPARATE}[args.dq]
    stream = torch.cuda.current_stream()

    if fwd_only:
        stages = ("fwd",)
    elif sparse:
        # block-sparse: each stage is one entry point (mask packing + forward;
        # mask packing + prep + fused backward)
        stages = ("fwd", "main")
        mask_dev = torch.from_numpy(mask_np).to(dev)
        ws_f = torch.empty(fa.fa_fwd_sparse_workspace_size(B, H, N, 0), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(fa.fa_bwd_sparse_workspace_size(B, H, N, 0), dtype=torch.uint8, device=dev)
    else:
        stages = ("fwd", "prep", "main")

    def run(evs=None, only=None):
        """One step (or only the stage named by `only`); evs maps a stage name to the
        (start, end) events recorded around it."""
        evs = evs or {}
        for name in (stages if only is None else (only,)):
            if name in evs: evs[name][0].record(stream)
            if fp8:
                fa.fa_fwd_fp8(q, k, v, o, lse, causal, scale, 1.0, 1.0, 1.0, stream)
            elif sparse and name == "fwd":
                fa.fa_fwd_sparse(q, k, v, o, lse, mask_dev, causal, scale, ws_f, stream)
            elif sparse:
                fa.fa_bwd_sparse(q, k, v, o, do, lse, dq, dk, dv, mask_dev, causal, scale, ws_b, stream)
            elif name == "fwd":
                fa.fa_fwd(q, k, v, o, lse, causal, scale, stream)
            elif name == "prep":
                fa.fa_bwd_prep(o, do, lse, ws, strategy, stream)
            else:
                fa.fa_bwd_main(q, k, v, o, do, lse, dq, dk, dv, ws, causal, scale, strategy, stream)
            if name in evs: evs[name][1].record(stream)

    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    K = args.steps
    # Stage breakdown: every launch bracketed by events (the events themselves
    # add a few microseconds per step, so this pass does not set the step time).
    brk = [{name: ev_pair() for name in stages} for _ in range(K)]
    for i in range(K):
        run(brk[i])
    torch.cuda.synchronize()
    stage_ms = {name: statistics.mean(e[name][0].elapsed_time(e[name][1]) for e in brk) for name in stages}
    dom = "main" if "main" in stage_ms and stage_ms["main"] >= stage_ms["fwd"] else "fwd"

    # Dominant kernel: a pass of K steps with events around its launches only,
    # which gives its average launch duration for the roofline entry (the
    # figure includes the dispatch gap in front of each launch).
    dom_ev = [{dom: ev_pair()} for _ in range(K)]
    for i in range(K):
        run(dom_ev[i])
    torch.cuda.synchronize()
    dom_ms = statistics.mean(e[dom][0].elapsed_time(e[dom][1]) for e in dom_ev)
    # the same kernel launched K times back to back between two events (its inputs
    # as the step leaves them): the launch duration plus the gap between queued launches
    b2b = ev_pair()
    b2b[0].record(stream)
    for i in range(K):
        run(only=dom)
    b2b[1].record(stream)
    torch.cuda.synchronize()
    dom_b2b_ms = b2b[0].elapsed_time(b2b[1]) / K

    # Timed region: K whole steps between two events, nothing else inside.
    t_start, t_end = ev_pair()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        run()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / K

    step_rule = "fwd" if fwd_only else "step"
    tf_step = flops(w, step_rule) / (ms_step * 1e-3) / 1e12
    tf_fwd = flops(w, "fwd") / (stage_ms["fwd"] * 1e-3) / 1e12
    bwd_ms = stage_ms.get("prep", 0.0) + stage_ms.get("main", 0.0)
    tf_bwd = flops(w, "bwd") / (bwd_ms * 1e-3) / 1e12 if bwd_ms > 0 else None
    fp32 = w["dtype"] == "fp32"
    peak = PEAK_FP32_TFLOPS if fp32 else PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS

    # roofline of the dominant kernel: algorithmic FLOP per launch / its average duration
    dom_flop = flops(w, "bwd") if dom == "main" else flops(w, "fwd")
    dom_tf = dom_flop / (dom_ms * 1e-3) / 1e12
    single = not (dom == "main" and (args.dq == "atomic" or fp32))
    roofline = {
        "bound": "mfma", "achieved": round(dom_tf, 2), "peak": peak, "unit": "TFLOP/s",
        "frac": round(dom_tf / peak, 4), "traffic": traffic_bytes(args.workload, dom) if args.dq == "default" else None,
        "traffic_unit": "bytes per launch beyond L2 (copy-calibrated FETCH_SIZE + WRITE_SIZE)",
        "algorithmic_bytes": algorithmic_bytes(w, dom),
        "kernel": (("bwd128_fused_kernel" if d == 128 else KERNELS[dom]) if dom == "main" else KERNELS[dom]) if single
                  else f"fa_bwd_main ({'atomic main + convert' if not fp32 else 'fp32'})",
        "flop_per_launch": dom_flop, "avg_launch_ms": round(dom_ms, 5),
        "avg_launch_source": "HIP events around the kernel's launches in a pass of K steps of their own, "
                             "outside the timed region (includes the dispatch gap in front of each launch)",
        "flop_rule": "fwd 4*B*H*N^2*d, bwd 10*B*H*N^2*d (five products), halved for causal",
    }
    if fp8:
        roofline.update({"traffic": None, "algorithmic_bytes": None, "kernel": "fwd_fp8_kernel",
                         "flop_rule": "fwd 4*B*H*N^2*d, halved for causal; peak: dense fp8 MFMA"})
    if sparse:
        roofline.update({
            "traffic": None, "algorithmic_bytes": None,
            "kernel": ("fa_bwd_sparse: mask packing + bwd_prep_kernel + " + ("bwd128_fused_kernel" if d == 128 else "bwd_fused_kernel")
                       + " (sparse)" if dom == "main"
                       else "fa_fwd_sparse: mask packing + fwd_kernel (sparse)"),
            "flop_rule": "fwd 4*B*H*d, bwd 10*B*H*d, per query-key pair kept by the block mask",
        })

    cold = None
    if args.flush_mall:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_ms = []
        for i in range(K):
            scratch.fill_(i & 0xFF)
            e0, e1 = ev_pair()
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            cold_ms.append(e0.elapsed_time(e1))
        del scratch
        cms = statistics.median(cold_ms)
        cold = {"ms_per_step_median": round(cms, 5), "ms_min": round(min(cold_ms), 5), "ms_max": round(max(cold_ms), 5),
                "tflops": round(flops(w, step_rule) / (cms * 1e-3) / 1e12, 3),
                "note": "each step after a 512 MiB scratch write; events around each step"}

    sclk = None
    if not args.no_sclk:
        def many():
            for _ in range(200):
                run()
        sclk = sclk_during(many)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, shape, scale, causal)

    cfg = {"workload": args.workload, "B": B, "H": H, "N": N, "d": d, "causal": causal, "dtype": w["dtype"],
           "scale": scale, "dq_strategy": args.dq}
    if sparse:
        cfg.update({"block": SPARSE_BLOCK, "density": w["sparse"]["density"], "mask_seed": w["sparse"]["mask_seed"],
                    "kept_blocks": int(mask_np.sum()), "blocks": int(mask_np.size),
                    "kept_pairs_per_head": w["pairs"]})
    out = {
        "metric": ("attention TFLOP/s fwd+bwd (10*B*H*d per kept query-key pair)" if sparse else
                   "attention TFLOP/s fwd, fp8 inputs (4*B*H*N^2*d, halved for causal)" if fp8 else
                   "attention TFLOP/s fwd (4*B*H*N^2*d, halved for causal)" if fwd_only else
                   "attention TFLOP/s fwd+bwd (10*B*H*N^2*d, halved for causal)"),
        "value": round(tf_step, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w["dtype"], "data": "synthetic: seeded i.i.d. N(0,1) inputs of the workload's shape",
        "config": cfg,
        "stage_breakdown": "per-stage means from a separate pass with events around every launch",
        "fwd": {"ms": round(stage_ms["fwd"], 5), "tflops": round(tf_fwd, 3), "frac_peak": round(tf_fwd / peak, 4)},
        "bwd": None if fwd_only else {"ms": round(bwd_ms, 5), "prep_ms": round(stage_ms.get("prep", 0.0), 5),
                                      "main_ms": round(stage_ms["main"], 5), "tflops_10x": round(tf_bwd, 3)},
        "fwd_bwd": None if fwd_only else {
            "tflops_10x": round(tf_step, 3), "frac_peak": round(tf_step / peak, 4),
            "tflops_14x_algorithmic": round(flops(w, "step_alg") / (ms_step * 1e-3) / 1e12, 3)},
        "io_fwd": {"flash_bytes": io_bytes(w)[0], "standard_bytes": io_bytes(w)[1],
                   "standard_over_flash": round(io_bytes(w)[1] / io_bytes(w)[0], 2)},
        "roofline": roofline, "cpu_baseline": cpu, "wall_s_timed": round(wall, 4),
        "dominant_launch_ms": {"median": round(statistics.median(e[dom][0].elapsed_time(e[dom][1]) for e in dom_ev), 5),
                               "min": round(min(e[dom][0].elapsed_time(e[dom][1]) for e in dom_ev), 5),
                               "max": round(max(e[dom][0].elapsed_time(e[dom][1]) for e in dom_ev), 5),
                               "back_to_back": round(dom_b2b_ms, 5)},
        "cold": cold, "sclk": sclk,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
