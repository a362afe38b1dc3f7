#!/usr/bin/env python3
"""Benchmark of the block-sparse attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input: the
pattern (log-linear rule or block mask -> CSR, built on the host and uploaded
once, then served from a device-resident cache as a model would for every
layer and step) and one fused forward launch.  Inputs are resident in HBM
before the timed region.  The K timed steps are captured in one HIP graph and
replayed (the forward of a single (B=1, H=8) batch lasts a few microseconds,
so eager launches would time the host, not the GPU); the eager rate is
reported beside it.

Prints ONE JSON line.  Metric: effective TFLOP/s over the selected blocks,
4 * bs^2 * d flop per selected block pair per (batch, head).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (selected blocks) + % bf16 MFMA peak, N=4096 log-linear"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_csr_amd", "csrc", "forward.hip")
DECODE_SRC = os.path.join(ROOT, "block_sparse_attention_csr_amd", "csrc", "decode.hip")
BACKWARD_SRC = os.path.join(ROOT, "block_sparse_attention_csr_amd", "csrc", "backward.hip")
PROFILES = os.path.join(ROOT, "profiles")
DECODE_METRIC = "decode GB/s (algorithmic bytes: visible K/V rows) + % of 8 TB/s HBM peak"


SHARED_SRC = os.path.join(ROOT, "block_sparse_attention_csr_amd", "csrc", "mfma_tiles.h")


def kernel_source_hash(path: str = KERNEL_SRC) -> str:
    """First 16 hex digits of the SHA-256 over a kernel's source file followed
    by the device header every kernel file includes (mfma_tiles.h), so that a
    profile record goes stale when either changes."""
    h = hashlib.sha256()
    for p in (path, SHARED_SRC):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="worked_example")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-graph", action="store_true", help="time eager launches only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cold", action="store_true",
                   help="skip the cold-cache launches (512 MiB write before each)")
    p.add_argument("--cold-launches", type=int, default=50)
    p.add_argument("--no-row-split", action="store_true",
                   help="walk every row in one workgroup (no bsa_forward_split)")
    p.add_argument("--no-saturating", action="store_true",
                   help="skip the B=32 line of the worked-example shape")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time for the oracle baseline")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured dense-GEMM and copy ceilings")
    p.add_argument("--causal", action="store_true",
                   help="time the causal forward (keys after each query hidden; the pattern "
                        "built causal) instead of the plain one")
    p.add_argument("--int8-kv", action="store_true",
                   help="decode on the int8 cache (bsa_decode_int8kv) for a decode workload; "
                        "the forward on int8 K/V (bsa_forward_int8kv) for a forward one")
    p.add_argument("--backward", action="store_true",
                   help="time the backward (dQ, dK, dV) of the workload instead of its forward")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run 5 device-to-device copies of 1 GiB (reference kernel for "
                        "scaling HBM byte counters) and exit")
    return p.parse_args(argv)


def copy_calibration():
    """Five 1 GiB device copies: each reads 1 GiB and writes 1 GiB of HBM.
    Profiled with FETCH_SIZE / WRITE_SIZE it gives the counter-to-bytes factor."""
    import torch

    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": 1 << 30,
                                           "bytes_written_per_copy": 1 << 30, "copies": 5}}))
    return 0


class Case:
    """Inputs, cached pattern and preallocated outputs of one workload."""

    def __init__(self, name, seed, device, causal=False, row_split=True):
        import numpy as np
        import torch

        import block_sparse_attention_csr_amd as bsa
        from synthetic_inputs import WORKLOADS, make_qkv, workload_block_mask

        self.bsa = bsa
        self.causal = causal
        self.row_split = row_split
        self.split = None
        self.workspace = None
        self.w = w = WORKLOADS[name]
        self.mask = workload_block_mask(w, seed)
        q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, seed)
        self.q, self.k, self.v = (t.to(device) for t in (q, k, v))
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=device)
        self.cache = bsa.PatternCache(device)
        if row_split:
            # long rows (a banded pattern's global rows) spread over workgroups;
            # plan and workspace made once, outside the timed steps
            self.split = self.cache.split_plan(w.N, w.block_size, mask=self.mask, causal=causal)
            if self.split is not None:
                need = bsa._load().bsa_row_split_workspace_bytes(w.B, w.H, w.block_size, w.d,
                                                                 self.split.n_items)
                self.workspace = torch.empty(need, dtype=torch.uint8, device=device)
        torch.cuda.synchronize()
        # First step: host pattern build + upload (cache miss) + forward.
        t0 = time.perf_counter()
        self.step()
        torch.cuda.synchronize()
        self.first_step_ms = (time.perf_counter() - t0) * 1e3
        self.nnz = self.cache.get(w.N, w.block_size, mask=self.mask, causal=causal)[2]
        # Selected (query, key) pairs: a whole block pair is bs^2 of them; with
        # causal masking a diagonal block keeps bs (bs + 1) / 2.
        pairs = float(w.block_size ** 2 * self.nnz)
        if causal:
            rp, ci = bsa.build_pattern(w.N, w.block_size, mask=self.mask, causal=True)
            rows = np.repeat(np.arange(w.M), np.diff(rp.numpy()))
            diag = int((ci.numpy() == rows).sum())
            pairs -= diag * (w.block_size ** 2 - w.block_size * (w.block_size + 1) // 2)
        self.flops = 4.0 * w.d * pairs * w.B * w.H
        elt = 2 if w.dtype == "bf16" else 4
        # compulsory traffic: Q, K, V read once, O written once, LSE written once
        self.compulsory_bytes = 4.0 * w.B * w.H * w.N * w.d * elt + 4.0 * w.B * w.H * w.N

    def step(self):
        w = self.w
        row_ptr, col_idx, nnz = self.cache.get(w.N, w.block_size, mask=self.mask,
                                               causal=self.causal)
        self.bsa.forward(self.q, self.k, self.v, row_ptr, col_idx, w.block_size,
                         out=self.out, lse=self.lse, nnz=nnz, causal=self.causal,
                         split=self.split, workspace=self.workspace)


class Int8KvCase:
    """The forward on int8 K/V with per-block scales (bsa_forward_int8kv):
    the workload's K and V quantised once (bsa_quantize_kv, untimed); a step
    is one forward launch on the codes."""

    def __init__(self, name, seed, device, causal=False):
        import torch

        import block_sparse_attention_csr_amd as bsa
        from synthetic_inputs import WORKLOADS, make_qkv, workload_block_mask

        assert not causal
        self.bsa = bsa
        self.w = w = WORKLOADS[name]
        self.mask = workload_block_mask(w, seed)
        q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, seed)
        self.q = q.to(device)
        kd, vd = k.to(device), v.to(device)
        self.kc, self.ks = bsa.quantize_kv(kd, w.block_size)
        self.vc, self.vs = bsa.quantize_kv(vd, w.block_size)
        del kd, vd
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=device)
        rp, ci = bsa.build_pattern(w.N, w.block_size, mask=self.mask)
        self.rp, self.ci, self.nnz = rp.to(device), ci.to(device), int(ci.numel())
        torch.cuda.synchronize()
        self.flops = 4.0 * w.block_size ** 2 * w.d * self.nnz * w.B * w.H
        rows = w.B * w.H * w.N
        # Q read and O written in bf16, K and V read as int8 codes plus one
        # float32 scale per block each, LSE written
        self.compulsory_bytes = (2.0 * 2 + 2.0 * 1) * rows * w.d + 4.0 * rows \
            + 2.0 * 4 * w.B * w.H * w.M
        self.bf16_bytes = 4.0 * 2 * rows * w.d + 4.0 * rows
        self.split = None
        t0 = time.perf_counter()
        self.step()
        torch.cuda.synchronize()
        self.first_step_ms = (time.perf_counter() - t0) * 1e3

    def step(self):
        w = self.w
        self.bsa.forward_int8kv(self.q, self.kc, self.ks, self.vc, self.vs, self.rp, self.ci,
                                w.block_size, out=self.out, lse=self.lse, nnz=self.nnz)


class DecodeCase:
    """One decode step: a new token for each of B sequences against a KV cache
    of capacity N (cached lengths uniform on [1, N]), log-linear pattern."""

    def __init__(self, name, seed, device, int8=False):
        import numpy as np
        import torch

        import block_sparse_attention_csr_amd as bsa
        from synthetic_inputs import WORKLOADS, decode_lengths, make_decode_inputs

        self.bsa = bsa
        self.int8 = int8
        self.w = w = WORKLOADS[name]
        q, k, v = make_decode_inputs(w.B, w.H, w.N, w.d, w.torch_dtype, seed)
        lengths = decode_lengths(w.B, w.N, seed)
        self.q, self.k, self.v = (t.to(device) for t in (q, k, v))
        if int8:  # the cache as int8 codes + per-block scales (quantised once, untimed)
            self.kc, self.ks = bsa.quantize_kv(self.k, w.block_size)
            self.vc, self.vs = bsa.quantize_kv(self.v, w.block_size)
            del self.k, self.v
        self.lengths = lengths.to(device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.H), dtype=torch.float32, device=device)
        rp, ci = bsa.build_pattern(w.N, w.block_size)
        self.rp, self.ci, self.nnz = rp.to(device), ci.to(device), int(ci.numel())
        # Visible cached positions of each sequence's new token: the positions
        # <= t of the blocks j <= t // bs its pattern row selects.
        rp_h, ci_h = rp.numpy(), ci.numpy()
        visible = 0
        for L in lengths.tolist():
            t = L - 1
            i = t // w.block_size
            for j in ci_h[rp_h[i]:rp_h[i + 1]]:
                if j <= i:
                    visible += min(w.block_size, t - int(j) * w.block_size + 1)
        elt = 2 if w.dtype == "bf16" else 4
        kv_elt = 1 if int8 else elt
        self.visible_keys = visible
        # Algorithmic bytes: every visible K and V row read once (int8: plus the
        # two scales of each visible block), q read, O and LSE written; flop:
        # q.k and p.v per visible key.
        self.bytes = (2.0 * visible * w.H * w.d * kv_elt + 2.0 * w.B * w.H * w.d * elt
                      + 4.0 * w.B * w.H)
        if int8:
            blocks = 0
            for L in lengths.tolist():
                i = (L - 1) // w.block_size
                blocks += sum(1 for j in ci_h[rp_h[i]:rp_h[i + 1]] if j <= i)
            self.bytes += 8.0 * blocks * w.H
        self.flops = 4.0 * visible * w.H * w.d

    def step(self):
        w = self.w
        if self.int8:
            self.bsa.decode_int8kv(self.q, self.kc, self.ks, self.vc, self.vs, self.lengths,
                                   self.rp, self.ci, w.block_size, out=self.out, lse=self.lse,
                                   nnz=self.nnz)
        else:
            self.bsa.decode(self.q, self.k, self.v, self.lengths, self.rp, self.ci, w.block_size,
                            out=self.out, lse=self.lse, nnz=self.nnz)


def decode_line(name, args, device, int8=False):
    """A graph-timed decode step (bsa_decode, or bsa_decode_int8kv on an int8
    cache): HBM-bound, reported in GB/s of algorithmic bytes against the
    8 TB/s peak, and in tokens per second."""
    import torch

    case = DecodeCase(name, args.seed, device, int8=int8)
    for _ in range(5):
        case.step()
    steps = max(20, min(200, args.steps // 5))
    g_step, g_evt = time_graph(case, steps) if not args.no_graph else (None, None)
    launch = time_events_per_launch(case, steps)
    step_s = g_step if g_step is not None else time_eager(case, steps)
    kernel_s = g_evt if g_evt is not None else launch
    w = case.w
    gbps = case.bytes / kernel_s / 1e9
    traffic = load_traffic(name + ("_int8kv" if int8 else ""), "bsa_decode", DECODE_SRC)
    line = {
        "value": round(case.bytes / step_s / 1e9, 1),
        "unit": "GB/s",
        "tokens_per_s": round(w.B / step_s, 1),
        "ms_per_step": step_s * 1e3,
        "kernel_us": kernel_s * 1e6,
        "per_launch_event_us": launch * 1e6,
        "description": (w.description.replace(", bf16", ", bf16 query; int8 K/V cache with "
                                                "per-block float32 scales") if int8
                        else w.description),
        "visible_keys_summed_over_batch_per_head": case.visible_keys,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "traffic_over_algorithmic": None if traffic is None
                     else round(traffic / case.bytes, 3),
                     "kernel": "bsa_decode_kernel",
                     "kv_cache": "int8 + per-block float32 scales" if int8 else w.dtype,
                     "algorithmic_bytes_per_launch": case.bytes,
                     "algorithmic_flop_per_launch": case.flops},
    }
    del case
    torch.cuda.empty_cache()
    return line


def time_eager(case, steps):
    import torch

    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        case.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / steps


def time_graph(case, steps):
    """Capture `steps` forward launches in one HIP graph; replay once timed.
    Returns (wall seconds per step, event seconds per launch)."""
    import torch

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        case.step()  # pattern already cached: no host build, no upload inside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(steps):
            case.step()
    graph.replay()  # untimed warm replay
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    replay_stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(replay_stream)
    graph.replay()
    end.record(replay_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / steps, start.elapsed_time(end) * 1e-3 / steps


def time_events_per_launch(case, steps):
    """Average launch duration from HIP events bracketing every launch on the
    launch stream, with the stream held by a sleep kernel while the host
    enqueues (so the host's enqueue rate does not show up as GPU time)."""
    import torch

    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    for a, b in evs:
        a.record(stream)
        case.step()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) * 1e-3 / steps


def load_traffic(workload: str, prefix: str = "bsa_fwd", src: str = KERNEL_SRC):
    """HBM bytes per launch from committed rocprofv3 counter summaries, valid
    only while the kernel source is unchanged since the counters were taken."""
    path = os.path.join(PROFILES, f"{prefix}_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def load_mfma(workload: str, src: str = KERNEL_SRC):
    """Matrix-core flop per launch counted by rocprofv3 (SQ_INSTS_VALU_MFMA_MOPS_*,
    512 flop each) from committed summaries, valid only while the kernel
    source is unchanged since the counters were taken."""
    path = os.path.join(PROFILES, f"bsa_fwd_mfma_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    return rec.get("mfma_flop_per_launch")


def time_cold(case, launches: int, scratch_mib: int = 512):
    """Cold-cache launch durations: before each launch a fill kernel writes a
    scratch buffer larger than the L2s and the MALL together, then HIP events
    bracket the launch alone.  Returns the median seconds per launch."""
    import statistics

    import torch

    scratch = torch.empty(scratch_mib << 20, dtype=torch.uint8, device=case.q.device)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        scratch.fill_(i & 0xFF)
        a.record(stream)
        case.step()
        b.record(stream)
    torch.cuda.synchronize()
    del scratch
    return statistics.median(a.elapsed_time(b) for a, b in evs) * 1e-3


def cpu_baseline(workload: str, seed: int, min_seconds: float):
    """Time the float64 oracle as it stands on this host's cores over whole
    passes of the workload (or of a bounded head subset for large ones)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    from synthetic_inputs import WORKLOADS, make_qkv, workload_block_mask

    w = WORKLOADS[workload]
    mask = workload_block_mask(w, seed)
    if mask is None:
        mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(w.N, w.block_size))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    if len(heads) > 8:
        heads = heads[:8]
    Bs = max(b for b, _ in heads) + 1
    q, k, v = make_qkv(Bs, w.H, w.N, w.d, w.torch_dtype, seed)
    f = lambda t: t.float().numpy().astype(np.float64)
    qf, kf, vf = f(q), f(k), f(v)
    nnz = int((mask != 0).sum())
    flops_per_pass = 4.0 * w.block_size ** 2 * w.d * nnz * len(heads)
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.block_sparse_attention(qf, kf, vf, mask, w.block_size, heads=heads)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el * (passes + 1) / passes > 30.0:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": flops_per_pass * passes / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{workload}: {len(heads)} of {w.B * w.H} (batch, head) pairs, "
                   f"{passes} full passes, {el:.1f} s wall; float64 dense masked attention"),
        "host_affinity_cpus": len(os.sched_getaffinity(0)),
    }


def practical_ceilings():
    """Measured ceilings on this GPU beside the published peaks: a dense bf16
    GEMM through torch (hipBLASLt) and a 1 GiB device-to-device copy."""
    import torch

    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    start.record()
    for _ in range(reps):
        torch.matmul(a, b)
    end.record()
    torch.cuda.synchronize()
    gemm = 2.0 * n ** 3 * reps / (start.elapsed_time(end) * 1e-3) / 1e12
    del a, b
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    start.record()
    for _ in range(5):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    copy = 2.0 * (1 << 30) * 5 / (start.elapsed_time(end) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"dense_bf16_gemm_tflops": round(gemm, 1),
            "dense_bf16_gemm": "torch.matmul 8192^3 bf16, 10 reps",
            "device_copy_gbps": round(copy, 1),
            "device_copy": "1 GiB copy, read + write bytes, 5 reps"}


class BackwardCase:
    """One backward pass (dQ and D, then dK and dV) over a workload, with the
    forward's output and LSE computed once beforehand."""

    def __init__(self, name, seed, device, causal=False):
        import torch

        import block_sparse_attention_csr_amd as bsa
        from synthetic_inputs import make_qkv

        self.fwd = Case(name, seed, device, causal=causal)
        self.bsa = bsa
        w = self.fwd.w
        self.dout = make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, seed + 7)[0].to(device)
        rp, ci = bsa.build_pattern(w.N, w.block_size, mask=self.fwd.mask, causal=causal)
        cp, ri = bsa.transpose_pattern(rp, ci)
        self.pat = [t.to(device) for t in (rp, ci, cp, ri)]
        # longest-first block orders of the CSR and the CSC (host, once)
        self.orders = [bsa.pattern_order(t).to(device) for t in (rp, cp)]
        self.grads = [torch.empty_like(self.fwd.q) for _ in range(3)]
        self.delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=device)
        self.fwd.step()
        torch.cuda.synchronize()
        # five products per selected pair (S recomputed, dP, dV, dQ, dK count as
        # the standard 2.5x of the forward's two)
        self.flops = 2.5 * self.fwd.flops
        self.compulsory_bytes = 2.0 * self.fwd.compulsory_bytes

    def step(self):
        f = self.fwd
        dq, dk, dv = self.grads
        self.bsa.backward(f.q, f.k, f.v, f.out, f.lse, self.dout, *self.pat, f.w.block_size,
                          causal=f.causal, dq=dq, dk=dk, dv=dv, delta=self.delta,
                          row_order=self.orders[0], col_order=self.orders[1])


TRAFFIC_NOTE = ("rocprofv3 FETCH_SIZE + WRITE_SIZE per launch: FETCH_SIZE counts L2-to-fabric "
                "requests, MALL (last-level cache) hits included, so it is an upper bound on "
                "HBM reads; each counter is scaled by what it reads for a 1 GiB device copy "
                "(x2 for FETCH_SIZE, x1 for WRITE_SIZE)")


def roofline_of(flops, compulsory_bytes, kernel_s, peak_flops, traffic, mfma_counted, kernel):
    """Roofline record of one forward step: the bound follows the arithmetic
    intensity of the algorithmic work against its compulsory HBM bytes,
    compared with the machine balance (peak flop / 8 TB/s)."""
    tflops = flops / kernel_s / 1e12
    gbps = compulsory_bytes / kernel_s / 1e9
    intensity = flops / compulsory_bytes
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(tflops / peak_flops, 4)}
    roof.update({
        "traffic": traffic,
        "kernel": kernel,
        "kernel_us": kernel_s * 1e6,
        "algorithmic_flop_per_launch": flops,
        "algorithmic_bytes_per_launch": compulsory_bytes,
        "intensity_flop_per_byte": round(intensity, 1),
        "ridge_flop_per_byte": round(ridge, 1),
        "mfma_achieved_tflops": round(tflops, 3),
        "mfma_frac": round(tflops / peak_flops, 4),
        "hbm_gbps_compulsory": round(gbps, 1),
        "hbm_frac_compulsory": round(gbps / PEAK_HBM_GBPS, 4),
        "traffic_over_algorithmic": None if traffic is None
        else round(traffic / compulsory_bytes, 3),
        "traffic_note": TRAFFIC_NOTE,
        "mfma_flop_counted_per_launch": mfma_counted,
        "mfma_counted_over_algorithmic": None if mfma_counted is None
        else round(mfma_counted / flops, 4),
    })
    return roof


def workload_line(name, args, device):
    """A graph-timed line for one of the other forward workloads
    (local+global with its heavy rows split, random mask, long), with the
    headline's fields: value, kernel_us, % of peak, roofline, traffic and
    counted MFMA work from the committed rocprofv3 records."""
    import torch

    case = Case(name, args.seed, device, row_split=not args.no_row_split)
    for _ in range(5):
        case.step()
    steps = max(10, min(100, args.steps // 10))
    g_step, g_evt = time_graph(case, steps) if not args.no_graph else (None, None)
    launch = time_events_per_launch(case, steps)
    step_s = g_step if g_step is not None else time_eager(case, steps)
    kernel_s = g_evt if g_evt is not None else launch
    w = case.w
    split = case.split is not None
    kernel = ("bsa_fwd_kernel (main pass) + bsa_fwd_kernel (split items) + bsa_fwd_merge_kernel"
              if split else "bsa_fwd_kernel")
    line = {
        "value": round(case.flops / step_s / 1e12, 3),
        "unit": "TFLOP/s",
        "ms_per_step": step_s * 1e3,
        "pct_bf16_mfma_peak": round(100.0 * case.flops / step_s / 1e12 / PEAK_BF16_TFLOPS, 2),
        "kernel_us": kernel_s * 1e6,
        "per_launch_event_us": launch * 1e6,
        "description": w.description,
        "nnz_per_head": case.nnz,
        "row_split": None if not split else {
            "heavy_rows_per_head": case.split.n_rows, "items_per_head": case.split.n_items,
            "launches_per_step": 3},
        "roofline": roofline_of(case.flops, case.compulsory_bytes, kernel_s, PEAK_BF16_TFLOPS,
                                load_traffic(name), load_mfma(name), kernel),
    }
    del case
    torch.cuda.empty_cache()
    return line


def side_line(name, args, device, causal, backward=False, int8_kv=False):
    """A graph-timed line for another workload (the saturating B = 32 shape,
    its causal forward, its backward or its forward on int8 K/V) reported
    beside the headline."""
    import torch

    cls = BackwardCase if backward else Int8KvCase if int8_kv else Case
    sat = cls(name, args.seed, device, causal=causal)
    for _ in range(5):
        sat.step()
    sat_steps = max(10, min(100, args.steps // 10))
    s_graph, s_evt = time_graph(sat, sat_steps) if not args.no_graph else (None, None)
    s_launch = time_events_per_launch(sat, sat_steps)
    s_step = s_graph if s_graph is not None else time_eager(sat, sat_steps)
    s_kernel = s_evt if s_evt is not None else s_launch
    record = name + ("_int8kv" if int8_kv else "")
    s_traffic = (None if causal else load_traffic(record, "bsa_bwd", BACKWARD_SRC) if backward
                 else load_traffic(record))
    s_mfma = None if causal or backward else load_mfma(record)
    line = {
        "value": round(sat.flops / s_step / 1e12, 3),
        "unit": "TFLOP/s",
        "ms_per_step": s_step * 1e3,
        "pct_bf16_mfma_peak": round(100.0 * sat.flops / s_step / 1e12 / PEAK_BF16_TFLOPS, 2),
        "kernel_us": s_kernel * 1e6,
        "mfma_achieved_tflops": round(sat.flops / s_kernel / 1e12, 3),
        "compulsory_hbm_gbps": round(sat.compulsory_bytes / s_kernel / 1e9, 1),
        "traffic": s_traffic,
        "traffic_over_algorithmic": None if s_traffic is None
        else round(s_traffic / sat.compulsory_bytes, 3),
    }
    if int8_kv:
        line["kv"] = "int8 codes + one float32 scale per block (bsa_quantize_kv), converted to bf16 in LDS"
        line["compulsory_bytes_per_launch"] = sat.compulsory_bytes
        line["bytes_vs_bf16_kv"] = round(sat.compulsory_bytes / sat.bf16_bytes, 4)
        line["roofline"] = roofline_of(sat.flops, sat.compulsory_bytes, s_kernel,
                                       PEAK_BF16_TFLOPS, s_traffic, s_mfma,
                                       "bsa_fwd_kernel (int8 K/V)")
    elif not backward and not causal:
        line["mfma_flop_counted_per_launch"] = s_mfma
        line["mfma_counted_over_algorithmic"] = (None if s_mfma is None
                                                 else round(s_mfma / sat.flops, 4))
        line["roofline"] = roofline_of(sat.flops, sat.compulsory_bytes, s_kernel,
                                       PEAK_BF16_TFLOPS, s_traffic, s_mfma, "bsa_fwd_kernel")
    if causal:
        line["flop_counting"] = "selected (query, key) pairs: diagonal blocks count bs(bs+1)/2"
    if backward:
        line["flop_counting"] = ("2.5x the forward's selected-pair flop (five products per pair: "
                                 "S, dP, dV, dQ, dK); two kernels per step")
    del sat
    torch.cuda.empty_cache()
    return line


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the forward shards over (batch, head) with no communication, so the N-GPU "
              "rate is N times the one-GPU rate of the per-GPU share.", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        return copy_calibration()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)

    if args.workload.startswith("decode"):
        # A decode workload on its own (profiling and side measurements).
        line = decode_line(args.workload, args, device, int8=args.int8_kv)
        from synthetic_inputs import WORKLOADS

        w = WORKLOADS[args.workload]
        print(json.dumps({
            "metric": DECODE_METRIC, "value": line.pop("value"), "unit": line.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": line.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded)",
            "config": {"workload": w.name, "description": line.pop("description"),
                       "kv_cache": "int8" if args.int8_kv else w.dtype},
            **line}), flush=True)
        return 0

    if args.backward:
        # The backward of a forward workload on its own (profiling).
        line = side_line(args.workload, args, device, causal=args.causal, backward=True)
        from synthetic_inputs import WORKLOADS

        w = WORKLOADS[args.workload]
        print(json.dumps({
            "metric": "backward " + METRIC, "value": line.pop("value"), "unit": line.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": line.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded)",
            "config": {"workload": w.name, "description": w.description, "pass": "backward"},
            **line}), flush=True)
        return 0
    if args.int8_kv:
        case = Int8KvCase(args.workload, args.seed, device)
    else:
        case = Case(args.workload, args.seed, device, causal=args.causal,
                    row_split=not args.no_row_split)
    w = case.w
    for _ in range(args.warmup):
        case.step()
    torch.cuda.synchronize()

    eager_s = time_eager(case, min(args.steps, 200))
    graph_s, graph_evt_s = (None, None)
    if not args.no_graph:
        try:
            graph_s, graph_evt_s = time_graph(case, args.steps)
        except Exception as e:  # graph capture unsupported: report eager only
            print(f"bench.py: graph timing unavailable ({e}); eager only", file=sys.stderr)
    launch_s = time_events_per_launch(case, min(args.steps, 200))
    step_s = graph_s if graph_s is not None else eager_s

    peak_flops = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    value = case.flops / step_s / 1e12
    # Kernel duration: HIP events around the graph replay on its stream (the
    # launches run back to back), else the per-launch event pairs.
    kernel_s = graph_evt_s if graph_evt_s is not None else launch_s
    record = args.workload + ("_int8kv" if args.int8_kv else "")
    traffic = None if args.causal else load_traffic(record)
    mfma_counted = None if args.causal else load_mfma(record)
    roof = roofline_of(case.flops, case.compulsory_bytes, kernel_s, peak_flops, traffic,
                       mfma_counted, "bsa_fwd_kernel (int8 K/V)" if args.int8_kv
                       else "bsa_fwd_kernel")
    roof["per_launch_event_us"] = launch_s * 1e6
    if args.workload == "worked_example":
        # 16.9 MB of inputs and outputs stay in the L2s and the 256 MB MALL
        # between back-to-back launches: the warm figure is not an HBM rate.
        roof["regime"] = ("latency: 1024 one-block workgroups of about 10 dependent 32x32 "
                          "entries each; the working set stays in L2/MALL between launches, so "
                          "the HBM fraction of this shape is the cold_cache line's")
    # Cold caches: a 512 MiB write before every launch (no L2 or MALL hits on
    # the inputs); each launch timed alone.
    cold = None
    if not args.no_cold:
        cold_s = time_cold(case, args.cold_launches)
        cold = {"kernel_us_median": cold_s * 1e6, "value": round(case.flops / cold_s / 1e12, 3),
                "unit": "TFLOP/s", "launches": args.cold_launches, "scratch_mib": 512,
                "compulsory_hbm_gbps": round(case.compulsory_bytes / cold_s / 1e9, 1),
                "hbm_frac": round(case.compulsory_bytes / cold_s / 1e9 / PEAK_HBM_GBPS, 4),
                "warm_per_launch_event_us": launch_s * 1e6,
                "timing": "HIP events around each launch alone (compare warm_per_launch_event_us, "
                          "timed the same way)"}
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V; pattern per workload)",
        "config": {
            "workload": w.name, "description": w.description, "B": w.B, "H": w.H, "N": w.N,
            "d": w.d, "block_size": w.block_size, "nnz_per_head": case.nnz,
            "pattern": w.pattern, "causal": bool(args.causal), "parallelism": "single GPU",
            "kv": "int8 codes + per-block float32 scales" if args.int8_kv else w.dtype,
            "timing": "HIP graph of K launches" if graph_s is not None else "eager",
            "row_split": None if case.split is None else {
                "heavy_rows_per_head": case.split.n_rows, "items_per_head": case.split.n_items,
                "launches_per_step": 3},
        },
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "eager_ms_per_step": eager_s * 1e3,
        "first_step_ms_with_pattern_build_and_upload": case.first_step_ms,
        "roofline": roof,
    }
    if cold is not None:
        result["cold_cache"] = cold

    if not args.no_saturating and args.workload == "worked_example" and not args.causal:
        del case
        torch.cuda.empty_cache()
        # The same shape with B = 32 fills the GPU; then its causal forward.
        result["saturating_worked_example_b32"] = side_line("worked_example_b32", args, device,
                                                            causal=False)
        result["causal_worked_example_b32"] = side_line("worked_example_b32", args, device,
                                                        causal=True)
        result["backward_worked_example_b32"] = side_line("worked_example_b32", args, device,
                                                          causal=False, backward=True)
        result["int8kv_worked_example_b32"] = side_line("worked_example_b32", args, device,
                                                        causal=False, int8_kv=True)
        for name in ("local_global", "random_mask", "long"):
            result[name] = workload_line(name, args, device)
        result["decode_worked_example"] = decode_line("decode_worked_example", args, device)
        result["decode_long"] = decode_line("decode_long", args, device)
        result["decode_worked_example_int8kv"] = decode_line("decode_worked_example", args,
                                                             device, int8=True)
        result["decode_long_int8kv"] = decode_line("decode_long", args, device, int8=True)

    if not args.no_ceilings:
        result["practical_ceilings"] = practical_ceilings()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload, args.seed, args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
