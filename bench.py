"""Benchmark of the FP8 fine-grained-scaled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --summarize DIR [--workload NAME]      (rocprofv3 CSVs -> profiles/)
    python bench.py --copy-probe BYTES                     (plain copy: counter calibration)

Default workload (the headline): the contiguous MoE GEMM, 8 experts x 4096
rows, N = 4096, K = 7168 (1.92 TFLOP per step, the largest single-GPU
configuration).  Other workloads: ``dense_m4096`` (five dense GEMMs at
M = 4096), ``dense_small_m`` (decode, M = 64 and 128), ``masked_16x256``
(MoE decode, 16 experts of capacity 256), ``dense_small`` (128x256x512).

Inputs are seeded synthetic N(0,1) fp32 matrices (``synth``), cast to e4m3
with the library's own cast kernels and kept resident in HBM; a *step* is one
pass over every GEMM of the workload.  MFMA-bound workloads are timed per
launch with HIP events on the stream the GEMMs are launched on; the
memory-bound ones (whose GPU time is below the host's per-call cost) by
replaying a HIP graph of whole steps, with weight copies rotated beyond the
256 MB last-level cache so every launch reads its weights from HBM.

One JSON line is printed: the aggregate throughput (``value``: algorithmic
flops / GEMM time), per-shape figures, a ``roofline`` object for the
dominant kernel (``traffic`` = measured HBM bytes per launch from the
committed counter summary of the same kernel sources, else null), a
``cpu_baseline`` (the CPU oracle on a bounded sample of the same workload)
and ``other_configs`` with per-shape figures of the other workloads and of
the UE8M0, addend, layout and K-grouped calls (skip with --no-other-configs).
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import moe_grouped_gemm_e4m3_amd as fg  # noqa: E402
import synth  # noqa: E402

PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "FP8 GEMM TFLOPS & GB/s (% of MI355X FP8 MFMA / HBM roofline) per shape"
CSRC = os.path.join(ROOT, "moe_grouped_gemm_e4m3_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = "contiguous_8x4096"
MALL_BYTES = 256e6


def progress(msg: str) -> None:
    """One line on stderr per finished phase (the JSON result goes to stdout)."""
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# Algorithmic work: what the method must compute and move (A and B once, the
# scale factors, D once, the row metadata), never what a kernel happens to do.

def dense_work(M, N, K):
    Kb, Nb = -(-K // 128), -(-N // 128)
    return 2 * M * N * K, M * K + N * K + 4 * (M * Kb + Nb * Kb) + 2 * M * N


def contiguous_work(rows_total, G, N, K):
    Kb, Nb = -(-K // 128), -(-N // 128)
    return (2 * rows_total * N * K,
            rows_total * K + G * N * K + 4 * (rows_total * Kb + G * Nb * Kb) + 2 * rows_total * N + 4 * rows_total)


def masked_work(mask, G, N, K):
    Kb, Nb = -(-K // 128), -(-N // 128)
    rv = int(np.sum(mask))
    gv = int(np.sum(np.asarray(mask) > 0))
    return 2 * rv * N * K, rv * K + gv * N * K + 4 * (rv * Kb + gv * Nb * Kb) + 2 * rv * N + 4 * G


# ---------------------------------------------------------------------------
# Resident problems.  Each has .launch(i) (one GEMM call; i picks a weight
# copy), .flops, .bytes, .shape and .label.

class Dense:
    def __init__(self, M, N, K, rotate=False, seed=0):
        self.shape, self.label = (M, N, K), "x".join(map(str, (M, N, K)))
        A32, B32 = synth.dense_problem(M, N, K, seed=seed)
        self.A32_cpu, self.B32_cpu = A32, B32
        self.a32 = A32.cuda()
        self.qa, self.sa = fg.fp8_cast_per_token(self.a32)
        self.qb, self.sb = fg.fp8_cast_per_block(B32.cuda())
        n_copies = max(1, int(2.5 * MALL_BYTES // (N * K))) if rotate else 0
        self.copies = [self.qb] + [self.qb.clone() for _ in range(n_copies)]
        self.D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        self.flops, self.bytes = dense_work(M, N, K)

    def launch(self, i=0):
        fg.gemm_fp8_nt(self.qa, self.sa, self.copies[i % len(self.copies)], self.sb, self.D)

    def cast(self):
        fg.fp8_cast_per_token(self.a32, self.qa, self.sa)


class Contiguous:
    def __init__(self, G, rows, N, K, seed=0):
        self.shape, self.label = (G, rows, N, K), f"{G}x{rows}x{N}x{K}"
        A32, B32, idx = synth.contiguous_problem([rows] * G, N, K, seed=seed)
        self.A32_cpu, self.B32_cpu, self.idx = A32, B32, idx
        self.qa, self.sa = fg.fp8_cast_per_token(A32.cuda())
        qb, sb = fg.fp8_cast_per_block(B32.reshape(G * N, K).cuda())
        self.qb, self.sb = qb.view(G, N, K), sb.view(G, -(-N // 128), -(-K // 128))
        self.mi = torch.from_numpy(idx.astype(np.int32)).cuda()
        self.D = torch.empty(idx.shape[0], N, dtype=torch.bfloat16, device="cuda")
        self.flops, self.bytes = contiguous_work(idx.shape[0], G, N, K)

    def launch(self, i=0):
        fg.gemm_fp8_grouped_contiguous(self.qa, self.sa, self.qb, self.sb, self.mi, self.D)


class Masked:
    def __init__(self, G, Mc, N, K, seed=0):
        self.shape, self.label = (G, Mc, N, K), f"{G}x{Mc}x{N}x{K}"
        A32, B32, mask = synth.masked_problem(G, Mc, N, K, seed=seed)
        self.mask = mask
        self.qa = torch.empty(G, Mc, K, dtype=torch.uint8, device="cuda")
        self.sa = fg.empty_activation_scales(Mc, K, groups=G)
        for g in range(G):
            fg.fp8_cast_per_token(A32[g].cuda(), self.qa[g], self.sa[g])
        qb, sb = fg.fp8_cast_per_block(B32.reshape(G * N, K).cuda())
        self.qb, self.sb = qb.view(G, N, K), sb.view(G, -(-N // 128), -(-K // 128))
        self.copies = [self.qb] + [self.qb.clone() for _ in range(max(1, int(2.8 * MALL_BYTES // (G * N * K))))]
        self.mt = torch.from_numpy(np.asarray(mask, np.int32)).cuda()
        self.D = torch.empty(G, Mc, N, dtype=torch.bfloat16, device="cuda")
        self.em = int(np.mean(mask))
        self.flops, self.bytes = masked_work(mask, G, N, K)

    def launch(self, i=0):
        fg.gemm_fp8_grouped_masked(self.qa, self.sa, self.copies[i % len(self.copies)], self.sb, self.mt, self.D,
                                   expected_m=self.em)


def build_workload(name):
    wl = synth.WORKLOADS[name]
    if wl.kind == "contiguous":
        return [Contiguous(*s) for s in wl.shapes], "mfma"
    if wl.kind == "masked":
        return [Masked(*s) for s in wl.shapes], "hbm"
    hbm = name == "dense_small_m" or name == "dense_small"
    return [Dense(*s, rotate=name == "dense_small_m") for s in wl.shapes], ("hbm" if hbm else "mfma")


# ---------------------------------------------------------------------------
# Launch log: with --launch-log PATH, every GEMM call of the workload (and
# every call a graph replay re-executes) is recorded in order as (problem
# index, "warm" | "timed"), so that the profile summaries can match the
# traced GEMM dispatches to shapes exactly (each call launches one GEMM
# kernel).

class LaunchLog:
    def __init__(self):
        self.on = False
        self.entries = []

    def add(self, seq, phase):
        if self.on:
            self.entries.extend((int(i), phase) for i in seq)

    def dump(self, path):
        with open(path, "w") as f:
            json.dump(self.entries, f)


LOG = LaunchLog()


# ---------------------------------------------------------------------------
# Timing

def event_steps(problems, steps, warmup):
    """Events around every launch on the launch stream; returns the wall time
    of the timed steps and the per-launch GPU ms [steps, problems]."""
    stream = torch.cuda.current_stream()
    for w in range(warmup):
        for pb in problems:
            pb.launch(w)
        LOG.add(range(len(problems)), "warm")
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in problems]
          for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        for i, pb in enumerate(problems):
            ev[s][i][0].record(stream)
            pb.launch(s)
            ev[s][i][1].record(stream)
        LOG.add(range(len(problems)), "timed")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, np.array([[a.elapsed_time(b) for (a, b) in row] for row in ev])


def graph_steps(problems, steps, warmup, per_graph=10):
    """Whole steps captured into a HIP graph (per_graph steps per graph) and
    replayed, so a step's time is GPU time, not the host's per-call cost.
    Returns the wall time of the timed replays and per-problem GPU ms per
    launch [reps, problems] from a graph per problem."""
    s = torch.cuda.Stream()
    step_seq = list(range(len(problems)))
    with torch.cuda.stream(s):
        for w in range(max(warmup, 1)):
            for pb in problems:
                pb.launch(w)
            LOG.add(step_seq, "warm")
    torch.cuda.synchronize()
    # the whole step, for the wall time
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for k in range(per_graph):
            for pb in problems:
                pb.launch(k)
    torch.cuda.synchronize()
    g.replay()
    LOG.add(step_seq * per_graph, "warm")
    torch.cuda.synchronize()
    reps = max(1, -(-steps // per_graph))
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
        LOG.add(step_seq * per_graph, "timed")
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * steps / (reps * per_graph)
    # per problem: one graph of per_graph launches each, timed by events
    per = []
    for i, pb in enumerate(problems):
        gp = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gp, stream=s):
            for k in range(per_graph):
                pb.launch(k)
        torch.cuda.synchronize()
        gp.replay()
        LOG.add([i] * per_graph, "warm")
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            gp.replay()
            b.record()
            LOG.add([i] * per_graph, "timed")
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / per_graph)
        per.append(ts)
        del gp
    del g
    return wall, np.array(per).T


def graph_time(launch, launches: int = 20, reps: int = 5) -> float:
    """GPU ms per launch of `launch(i)` by replay of a graph of `launches` calls."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for i in range(3):
            launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(launches):
            launch(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / launches)
    return float(np.median(ts))


def event_time(launch, reps: int = 10) -> float:
    """Median GPU ms of `launch()` over `reps` event-timed calls, after three untimed ones."""
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def shape_entry(config, shape, ms, flops, nbytes, bound):
    tf = flops / ms / 1e9
    gbs = nbytes / ms / 1e6
    return {"config": config, "shape": list(shape), "us": round(ms * 1e3, 2), "tflops": round(tf, 1),
            "pct_mfma": round(tf / PEAK_FP8_TFLOPS * 100, 1), "gbs": round(gbs, 1),
            "pct_hbm": round(gbs / PEAK_HBM_GBS * 100, 1), "bound": bound}


# ---------------------------------------------------------------------------
# Other configurations (per shape)

def other_configs(headline: str):
    out = []
    # the dense workloads (skipping the one that is the headline)
    for name in ("dense_small", "dense_m4096", "dense_small_m", "masked_16x256"):
        if name == headline:
            continue
        problems, bound = build_workload(name)
        if bound == "hbm":
            _, per = graph_steps(problems, 20, 3)
        else:
            _, per = event_steps(problems, 10, 3)
        tot_fl = tot_ms = 0.0
        for i, pb in enumerate(problems):
            ms = float(np.median(per[:, i]))
            out.append(shape_entry(name, pb.shape, ms, pb.flops, pb.bytes, bound if name != "dense_small" else "launch"))
            tot_fl += pb.flops
            tot_ms += ms
            progress(f"{name} {pb.label}: {ms * 1e3:.2f} us")
        if len(problems) > 1:
            e = shape_entry(name + "_aggregate", ["all"], tot_ms, tot_fl, sum(p.bytes for p in problems), bound)
            out.append(e)
        del problems
        torch.cuda.empty_cache()
    # dense M=4096 with power-of-two (UE8M0) factors
    for (M, N, K) in synth.DENSE_M4096.shapes:
        A32, B32 = synth.dense_problem(M, N, K, seed=0)
        qa, sa = fg.fp8_cast_per_token_ue8m0(A32.cuda())
        qb, sb = fg.fp8_cast_per_block_ue8m0(B32.cuda())
        del A32, B32
        D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ms = event_time(lambda: fg.gemm_fp8_nt_ue8m0(qa, sa, qb, sb, D))
        Kb4 = (K // 128 + 3) // 4
        nbytes = M * K + N * K + 4 * (M * Kb4 + -(-N // 128) * Kb4) + 2 * M * N
        out.append(shape_entry("dense_m4096_ue8m0", (M, N, K), ms, 2 * M * N * K, nbytes, "mfma"))
        del qa, qb, D
        progress(f"UE8M0 dense {M}x{N}x{K}: {ms * 1e3:.2f} us")
    # dense M=4096 with an fp32 addend (D = C + A B^T) and in the NN and TN
    # layouts, the plain GEMM on the same operands timed beside them
    for (M, N, K) in synth.DENSE_M4096.shapes:
        A32, B32 = synth.dense_problem(M, N, K, seed=0)
        qa, sa = fg.fp8_cast_per_token(A32.cuda())
        qb, sb = fg.fp8_cast_per_block(B32.cuda())
        del A32, B32
        C = torch.randn(M, N, generator=torch.Generator().manual_seed(1)).cuda()
        D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ms = event_time(lambda: fg.gemm_fp8_nt_c(qa, sa, qb, sb, C, D))
        plain = event_time(lambda: fg.gemm_fp8_nt(qa, sa, qb, sb, D))
        fl, nbytes = dense_work(M, N, K)
        e = shape_entry("dense_m4096_addend", (M, N, K), ms, fl, nbytes + 4 * M * N, "mfma")
        e["plain_us"] = round(plain * 1e3, 2)
        out.append(e)
        for layout in ("nn", "tn"):
            As = qa.t().contiguous() if layout[0] == "t" else qa
            Bs = qb.t().contiguous() if layout[1] == "n" else qb
            ws = torch.empty(fg.layout_workspace_bytes(layout, M, N, K), dtype=torch.uint8, device="cuda")
            gemm = getattr(fg, "gemm_fp8_" + layout)
            ms = event_time(lambda: gemm(As, sa, Bs, sb, D, workspace=ws))
            e = shape_entry("dense_m4096_" + layout, (M, N, K), ms, fl, nbytes, "mfma")
            e["plain_us"] = round(plain * 1e3, 2)
            out.append(e)
            del As, Bs, ws
        del qa, qb, C, D
        progress(f"addend and layouts {M}x{N}x{K} done")
    # K-grouped TN (weight gradients of the contiguous workload: 8 experts x
    # 4096 tokens, M = 4096, N = 7168)
    M, N, ks = 4096, 7168, [4096] * 8
    Kt = sum(ks)
    gen = torch.Generator(device="cuda").manual_seed(0)
    qa, sa = fg.fp8_cast_per_token(torch.randn(M, Kt, device="cuda", generator=gen))
    qb, sb = fg.fp8_cast_per_block(torch.randn(N, Kt, device="cuda", generator=gen))
    As, Bs = qa.t().contiguous(), qb.t().contiguous()
    del qa, qb
    D = torch.empty(len(ks), M, N, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(fg.k_grouped_workspace_bytes(M, N, Kt), dtype=torch.uint8, device="cuda")
    ms = event_time(lambda: fg.gemm_fp8_k_grouped_tn_contiguous(As, sa, Bs, sb, ks, D, workspace=ws), reps=5)
    Kb = Kt // 128
    nbytes = (M + N) * Kt + 4 * (M * Kb + -(-N // 128) * Kb) + 2 * len(ks) * M * N
    out.append(shape_entry("k_grouped_tn_8x4096", (len(ks), M, N, ks[0]), ms, 2 * M * N * Kt, nbytes, "mfma"))
    del As, Bs, D, ws
    progress(f"K-grouped TN: {ms * 1e3:.2f} us")
    # the contiguous and masked GEMMs with power-of-two (UE8M0) factors
    G, rows, N, K = synth.CONTIGUOUS_8x4096.shapes[0]
    A32, B32, idx = synth.contiguous_problem([rows] * G, N, K, seed=0)
    Mt = idx.shape[0]
    mi = torch.from_numpy(idx.astype(np.int32)).cuda()
    qa, sa = fg.fp8_cast_per_token_ue8m0(A32.cuda())
    qb, sb = fg.fp8_cast_per_block_ue8m0(B32.reshape(G * N, K).cuda())
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, -1)
    D = torch.empty(Mt, N, dtype=torch.bfloat16, device="cuda")
    ms = event_time(lambda: fg.gemm_fp8_grouped_contiguous_ue8m0(qa, sa, qb, sb, mi, D), reps=5)
    fl, nbytes = contiguous_work(Mt, G, N, K)
    out.append(shape_entry("contiguous_8x4096_ue8m0", (G, rows, N, K), ms, fl, nbytes, "mfma"))
    del A32, B32, qa, qb, D
    progress(f"contiguous ue8m0: {ms * 1e3:.2f} us")
    for (G, Mc, N, K) in synth.MASKED_16x256.shapes:
        A32, B32, mask = synth.masked_problem(G, Mc, N, K, seed=0)
        kb4 = (K // 128 + 3) // 4
        qa = torch.empty(G, Mc, K, dtype=torch.uint8, device="cuda")
        sa = torch.empty(G, kb4, fg.aligned_scale_ld(Mc), dtype=torch.int32, device="cuda")[:, :, :Mc]
        for g in range(G):
            fg.fp8_cast_per_token_ue8m0(A32[g].cuda(), qa[g], sa[g])
        qb, sb = fg.fp8_cast_per_block_ue8m0(B32.reshape(G * N, K).cuda())
        qb, sb = qb.view(G, N, K), sb.view(G, -(-N // 128), kb4)
        copies = [qb] + [qb.clone() for _ in range(max(1, int(2.8 * MALL_BYTES // (G * N * K))))]
        mt = torch.from_numpy(np.asarray(mask, np.int32)).cuda()
        D = torch.empty(G, Mc, N, dtype=torch.bfloat16, device="cuda")
        ms = graph_time(lambda i: fg.gemm_fp8_grouped_masked_ue8m0(qa, sa, copies[i % len(copies)], sb, mt, D),
                        launches=10)
        fl, nbytes = masked_work(mask, G, N, K)
        out.append(shape_entry("masked_16x256_ue8m0", (G, Mc, N, K), ms, fl, nbytes, "hbm"))
        del copies, qa, qb, D
        progress(f"masked ue8m0 {G}x{Mc}x{N}x{K}: {ms * 1e3:.2f} us")
    return out


def time_casts(problems):
    """Activation-cast GPU time per launch (graph replay)."""
    out = []
    for pb in problems:
        if not hasattr(pb, "cast"):
            continue
        ms = graph_time(lambda i, pb=pb: pb.cast())
        M, K = pb.shape[0], pb.shape[2]
        nbytes = M * K * 5 + 4 * M * (K // 128)
        out.append({"M": M, "K": K, "us": round(ms * 1e3, 2), "gbs": round(nbytes / ms / 1e6, 1),
                    "pct_hbm": round(nbytes / ms / 1e6 / PEAK_HBM_GBS * 100, 1)})
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle (fp64 blockwise GEMM) on a bounded sample

def cpu_baseline(problems, budget_s: float = 15.0):
    """The oracle on a bounded sample of the workload's outputs, at full K:
    dense, rows [0, 64) x columns [0, 256) of each shape; contiguous, rows
    [0, 64) of each expert x columns [0, 256) of that expert's weights;
    masked, the first min(count, 64) valid rows of every group x columns
    [0, 256).  The sample operands are quantised by the oracle's own
    quantiser.  Timed on every host BLAS thread."""
    from oracle import gemm as ogemm, quant

    try:
        from threadpoolctl import threadpool_info

        info = [t for t in threadpool_info() if t.get("user_api") == "blas"]
        cores = max([t.get("num_threads", 0) for t in info] or [0])
        blas = ", ".join(sorted({f"{t.get('internal_api')} {t.get('version')}" for t in info}))
    except Exception:  # pragma: no cover
        cores, blas = 0, ""
    cores = cores or len(os.sched_getaffinity(0))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    ms, ns = 64, 256
    samples = []
    what = ""
    for pb in problems:
        if isinstance(pb, Contiguous):
            G, rows, N, K = pb.shape
            A = pb.A32_cpu.numpy()
            B = pb.B32_cpu.numpy()
            for e in range(G):
                r0 = int(np.nonzero(pb.idx == e)[0][0])
                samples.append((A[r0:r0 + ms], B[e, :ns], K))
            what = f"rows [0, {ms}) of each of the {G} experts x columns [0, {ns}) of its weights"
        elif isinstance(pb, Masked):
            continue
        else:
            M, N, K = pb.shape
            samples.append((pb.A32_cpu.numpy()[:ms], pb.B32_cpu.numpy()[:ns], K))
            what = f"D[0:{ms}, 0:{ns}] of each of the {len(problems)} shapes"
    if not samples:  # masked workload: the first rows of every group
        for pb in problems:
            G, Mc, N, K = pb.shape
            A32, B32, mask = synth.masked_problem(G, Mc, N, K, seed=0)
            for g in range(G):
                r = min(int(mask[g]), ms)
                if r:
                    samples.append((A32[g, :r].numpy(), B32[g, :ns].numpy(), K))
        what = f"the first min(count, {ms}) valid rows of every group x columns [0, {ns})"
    qs = []
    for a, b, K in samples:
        qa, sa = quant.quantize_per_token(a)
        qb, sb = quant.quantize_per_block(b)
        qs.append((qa, sa, qb, sb, 2 * a.shape[0] * b.shape[0] * K))
    t0 = time.perf_counter()
    flops = 0
    for qa, sa, qb, sb, fl in qs:
        ogemm.gemm_nt(qa, sa, qb, sb)
        flops += fl
    dt = time.perf_counter() - t0
    reps = max(1, int(budget_s / max(dt, 1e-3)))
    t0 = time.perf_counter()
    for _ in range(reps):
        for qa, sa, qb, sb, _fl in qs:
            ogemm.gemm_nt(qa, sa, qb, sb)
    dt = time.perf_counter() - t0
    return {
        "value": round(flops * reps / dt / 1e12, 6),
        "unit": "TFLOPS",
        "cores": int(cores),
        "kind": "oracle",
        "cpu_model": cpu_model,
        "blas": blas,
        "sample": f"fp64 blockwise oracle on {what}, at full K; {reps} passes, {dt:.1f} s",
    }


def traffic_summary(workload: str):
    """The committed counter summary of the workload's GEMM kernel, if it was
    taken on the current kernel sources."""
    path = os.path.join(PROFILES, f"{workload}_traffic.json")
    try:
        with open(path) as f:
            summ = json.load(f)
    except OSError:
        return None
    if summ.get("kernel_source_hash") != kernel_source_hash():
        return None
    return summ


# ---------------------------------------------------------------------------
# rocprofv3 CSV -> profiles/ summaries

PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o run -- "
             "python3 bench.py --workload {w} --no-other-configs --no-cpu-baseline --steps {s} --warmup 2 "
             "--launch-log {d}/trace/launch_log.json",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o run -- "
             "python3 bench.py --workload {w} --no-other-configs --no-cpu-baseline --steps 2 --warmup 1 "
             "--launch-log {d}/fetch/launch_log.json",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o run -- "
             "python3 bench.py --workload {w} --no-other-configs --no-cpu-baseline --steps 2 --warmup 1 "
             "--launch-log {d}/write/launch_log.json",
    "mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F8 GRBM_GUI_ACTIVE --output-format csv "
            "-d {d}/mfma -o run -- python3 bench.py --workload {w} --no-other-configs --no-cpu-baseline --steps 2 --warmup 1 "
            "--launch-log {d}/mfma/launch_log.json",
    "copyf": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/copyf -o run -- python3 bench.py --copy-probe 1073741824",
    "copyw": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/copyw -o run -- python3 bench.py --copy-probe 1073741824",
}


def _csv(path_glob):
    files = sorted(glob.glob(path_glob, recursive=True))
    return files[0] if files else None


def _dispatches(path):
    """Kernel dispatches of a kernel-trace or counter-collection CSV, in
    dispatch order: name, grid, duration (us) and any counters."""
    d = collections.OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            i = int(r["Dispatch_Id"])
            if i not in d:
                grid = r.get("Grid_Size") or str(int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
                d[i] = {"name": r["Kernel_Name"], "grid": int(grid),
                        "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3}
            if "Counter_Name" in r:
                d[i][r["Counter_Name"]] = d[i].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [d[k] for k in sorted(d)]


def _gemm_dispatches(rows):
    return [r for r in rows if "gemm_fp8_" in r["name"]]


def _short(name):
    return name.split("(")[0].replace("void ", "")


def _per_shape(rows, n_shapes, log_path):
    """The GEMM dispatches of a run matched to its launch log (one entry per
    GEMM call, in order): the timed dispatches of each shape."""
    g = _gemm_dispatches(rows)
    with open(log_path) as f:
        log = json.load(f)
    if len(log) != len(g):
        raise SystemExit(f"{log_path}: {len(log)} logged GEMM calls but {len(g)} GEMM dispatches")
    out = [[] for _ in range(n_shapes)]
    for (i, phase), r in zip(log, g):
        if phase == "timed":
            out[i].append(r)
    return out


def _calibration(d):
    out = {}
    for key, ctr in (("copyf", "FETCH_SIZE"), ("copyw", "WRITE_SIZE")):
        p = _csv(os.path.join(d, key, "**", "*counter_collection.csv"))
        if not p:
            return None
        rows = [r for r in _dispatches(p) if ctr in r]
        big = max(rows, key=lambda r: r[ctr])  # the 1 GiB copy
        out[ctr] = {"kib_read": big[ctr], "factor": round((1 << 30) / 1024 / big[ctr], 4), "kernel": _short(big["name"])}
    return out


MAX_CLOCK_GHZ = 2.4  # MI355X peak shader clock


def summarize(d: str, workload: str, steps: int):
    """Write profiles/<workload>_summary.md (and _traffic.json) from the
    rocprofv3 runs under d (PROFILE_COMMANDS, with -d d/<key>)."""
    problems_shapes = synth.WORKLOADS[workload].shapes
    n = len(problems_shapes)
    trace = _csv(os.path.join(d, "trace", "**", "*kernel_trace.csv"))
    if not trace:
        raise SystemExit(f"no kernel trace under {d}/trace")
    h = kernel_source_hash()
    tr = _per_shape(_dispatches(trace), n, os.path.join(d, "trace", "launch_log.json"))
    cal = _calibration(d)
    ctr = {}
    for key in ("fetch", "write", "mfma"):
        p = _csv(os.path.join(d, key, "**", "*counter_collection.csv"))
        if p:
            ctr[key] = _per_shape(_dispatches(p), n, os.path.join(d, key, "launch_log.json"))
    work = []
    for s in problems_shapes:
        if len(s) == 3:
            work.append(dense_work(*s))
        elif synth.WORKLOADS[workload].kind == "contiguous":
            G, rows, N, K = s
            work.append(contiguous_work(G * rows, G, N, K))
        else:
            G, Mc, N, K = s
            work.append(masked_work(synth.masked_counts(G, Mc, 0), G, N, K))
    lines = [f"# {workload}: GEMM kernel durations, HBM traffic and MFMA counters", "",
             "Commands (one MI355X, from the repository root; `bench.py --summarize <dir> --workload "
             f"{workload}` wrote this file from their CSV output):", ""]
    for key in ("trace", "fetch", "write", "copyf", "copyw", "mfma"):
        lines.append(f"- `{PROFILE_COMMANDS[key].format(d='<dir>', w=workload, s=steps)}`")
    lines += ["", f"Kernel sources hash: `{h}` (sha256 over `moe_grouped_gemm_e4m3_amd/csrc`, as bench.py computes it).",
              "Durations are kernel-trace start/end times of the timed GEMM dispatches (the launch log that bench.py "
              "writes with --launch-log matches dispatches to shapes; warm-up calls are dropped).  "
              "HBM bytes are FETCH_SIZE and WRITE_SIZE per dispatch (KiB) scaled by what the same counters read "
              "for a plain 1 GiB device copy"
              + (f" (fetch x{cal['FETCH_SIZE']['factor']}, write x{cal['WRITE_SIZE']['factor']}; copy kernel "
                 f"`{cal['FETCH_SIZE']['kernel']}`)" if cal else " (no calibration runs found: raw x1)")
              + ", averaged over the counter runs' timed dispatches of the shape.", ""]
    head = "| shape | kernel | dispatches | avg us | TFLOP/s | % of 5.0 PF | algorithmic MB | GB/s (alg.) | % of 8 TB/s |"
    sep = "|---|---|---|---|---|---|---|---|---|"
    if "fetch" in ctr and "write" in ctr:
        head += " measured HBM MB | measured / algorithmic |"
        sep += "---|---|"
    if "mfma" in ctr:
        head += " clock GHz | MFMA busy | executed / algorithmic flops |"
        sep += "---|---|---|"
    lines += [head, sep]
    ff = cal["FETCH_SIZE"]["factor"] if cal else 1.0
    wf = cal["WRITE_SIZE"]["factor"] if cal else 1.0
    tot = {"us": 0.0, "flops": 0.0, "hbm": 0.0, "alg": 0.0, "n": 0}
    per_shape = []
    for i, s in enumerate(problems_shapes):
        rs = tr[i]
        us = float(np.mean([r["us"] for r in rs]))
        fl, nb = work[i]
        row = (f"| {'x'.join(map(str, s))} | `{_short(rs[0]['name'])}` | {len(rs)} | {us:.2f} | {fl / us / 1e6:.1f} | "
               f"{fl / us / 1e6 / 50:.1f} | {nb / 1e6:.1f} | {nb / us / 1e3:.1f} | {nb / us / 1e3 / 80:.1f} |")
        entry = {"shape": list(s), "kernel": _short(rs[0]["name"]), "avg_us": round(us, 3), "flops": fl,
                 "algorithmic_bytes": nb}
        if "fetch" in ctr and "write" in ctr:
            fb = float(np.mean([r["FETCH_SIZE"] for r in ctr["fetch"][i]])) * 1024 * ff
            wb = float(np.mean([r["WRITE_SIZE"] for r in ctr["write"][i]])) * 1024 * wf
            row += f" {(fb + wb) / 1e6:.1f} | {(fb + wb) / nb:.2f} |"
            entry.update(fetch_bytes=int(fb), write_bytes=int(wb), hbm_bytes=int(fb + wb))
            tot["hbm"] += fb + wb
        if "mfma" in ctr:
            ms_ = ctr["mfma"][i]
            gui = float(np.mean([r["GRBM_GUI_ACTIVE"] for r in ms_]))
            busy = float(np.mean([r["SQ_VALU_MFMA_BUSY_CYCLES"] for r in ms_]))
            mops = float(np.mean([r["SQ_INSTS_VALU_MFMA_MOPS_F8"] for r in ms_]))
            clk = gui / 8 / (us * 1e-6) / 1e9
            # the counter run's busy window per dispatch includes its launch
            # overhead: on launches of a few microseconds the ratio to the
            # traced duration overstates the clock, shown then as n/a
            clk_s = f"{clk:.2f}" if clk <= MAX_CLOCK_GHZ else "n/a"
            row += f" {clk_s} | {busy / (gui / 8 * 1024) * 100:.1f} % | {mops * 512 / fl:.3f} |"
        lines.append(row)
        per_shape.append(entry)
        tot["us"] += us
        tot["flops"] += fl
        tot["alg"] += nb
        tot["n"] += 1
    mean_us = tot["us"] / n
    lines += ["", f"Average launch over the {n} shape(s): {mean_us:.2f} us, {tot['flops'] / n:.4g} algorithmic flops, "
              f"{tot['flops'] / tot['us'] / 1e6:.1f} TFLOP/s ({tot['flops'] / tot['us'] / 1e6 / 50:.1f} % of 5.0 PFLOP/s)"
              + (f"; measured HBM bytes per launch {tot['hbm'] / n:.4g} = {tot['hbm'] / tot['alg']:.2f} x the "
                 f"algorithmic {tot['alg'] / n:.4g}." if tot["hbm"] else "."), ""]
    if "mfma" in ctr:
        lines += ["MFMA counters: `SQ_INSTS_VALU_MFMA_MOPS_F8` x 512 = FP8 flops executed; `GRBM_GUI_ACTIVE` / 8 "
                  "(XCDs) / duration = shader clock; `SQ_VALU_MFMA_BUSY_CYCLES` / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs) = "
                  "the fraction of SIMD cycles the matrix core was busy, at the clock the chip ran.  The clock is "
                  f"n/a where that ratio exceeds the chip's {MAX_CLOCK_GHZ} GHz: on short launches the counter run's "
                  "busy window includes the dispatch overhead.", ""]
    stats = _csv(os.path.join(d, "trace", "**", "*kernel_stats.csv"))
    if stats:
        lines += ["All kernels of the traced run (rocprofv3 --stats):", "",
                  "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
        with open(stats) as f:
            for r in csv.DictReader(f):
                lines.append(f"| `{_short(r['Name'])[:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                             f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                             f"{float(r['Percentage']):.1f} |")
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"{workload}_summary.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if tot["hbm"]:
        tj = {"workload": workload, "kernel_source_hash": h, "calibration": cal,
              "commands": [PROFILE_COMMANDS[k].format(d="<dir>", w=workload, s=steps)
                           for k in ("fetch", "write", "copyf", "copyw")],
              "per_shape": per_shape, "avg_us": round(mean_us, 3),
              "hbm_bytes_per_launch": int(tot["hbm"] / n), "algorithmic_bytes_per_launch": int(tot["alg"] / n)}
        with open(os.path.join(PROFILES, f"{workload}_traffic.json"), "w") as f:
            json.dump(tj, f, indent=1)
    print(f"wrote {workload}_summary.md" + (" and _traffic.json" if tot["hbm"] else "") + f" (hash {h})")


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true", help="time only the chosen workload")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 3 times (counter calibration)")
    ap.add_argument("--summarize", metavar="DIR", help="write profiles/ summaries from rocprofv3 CSVs under DIR")
    ap.add_argument("--launch-log", metavar="PATH", help="record every GEMM call of the workload (for --summarize)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.workload, args.steps)
        return
    if args.copy_probe:
        n = args.copy_probe // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1 (no multi-GPU path exists)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    fg.load_library()
    problems, bound = build_workload(args.workload)
    LOG.on = bool(args.launch_log)
    torch.cuda.synchronize()
    progress(f"{args.workload}: {len(problems)} problem(s) resident")
    if bound == "hbm":
        wall, per = graph_steps(problems, args.steps, args.warmup)
    else:
        wall, per = event_steps(problems, args.steps, args.warmup)
    progress(f"{args.steps} timed steps: {wall / args.steps * 1e3:.3f} ms per step")
    LOG.on = False
    if args.launch_log:
        os.makedirs(os.path.dirname(os.path.abspath(args.launch_log)), exist_ok=True)
        LOG.dump(args.launch_log)
    total_flops = sum(pb.flops for pb in problems)
    total_bytes = sum(pb.bytes for pb in problems)
    mean_ms = per.mean(axis=0)  # per problem
    step_ms = float(mean_ms.sum())
    value = total_flops / (step_ms * 1e-3) / 1e12
    shapes = [shape_entry(args.workload, pb.shape, float(mean_ms[i]), pb.flops, pb.bytes, bound)
              for i, pb in enumerate(problems)]
    casts = time_casts(problems) if args.workload.startswith("dense") else None
    others = None if args.no_other_configs else other_configs(args.workload)
    # roofline of the dominant kernel: algorithmic work per launch / mean launch time
    fl_per = total_flops / len(problems)
    by_per = total_bytes / len(problems)
    launch_ms = step_ms / len(problems)
    summ = traffic_summary(args.workload)
    if bound == "mfma":
        achieved, peak, unit = fl_per / launch_ms / 1e9, PEAK_FP8_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = by_per / launch_ms / 1e6, PEAK_HBM_GBS, "GB/s"
    kernel = {"contiguous": "gemm_fp8_big_kernel (contiguous)", "masked": "gemm_fp8_big_kernel (masked)"}.get(
        synth.WORKLOADS[args.workload].kind, "gemm_fp8_big_kernel / gemm_fp8_skinny_kernel (dense)")
    cfg = {"workload": args.workload, "shapes": [list(pb.shape) for pb in problems],
           "gemm_ms_per_step": round(step_ms, 4), "gbs": round(total_bytes / (step_ms * 1e-3) / 1e9, 1)}
    if isinstance(problems[0], Contiguous):
        G, rows, N, K = problems[0].shape
        cfg.update(experts=G, rows_per_expert=rows, N=N, K=K, m_total=rows * G)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": cfg,
        "shapes": shapes,
        "cast": casts,
        "other_configs": others,
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": summ["hbm_bytes_per_launch"] if summ else None,
            "kernel": kernel,
            "flops_per_launch": fl_per,
            "algorithmic_bytes_per_launch": by_per,
            "launch_us": round(launch_ms * 1e3, 2),
            "timing": "HIP events on the launch stream" if bound == "mfma" else "HIP graph replay, events",
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(problems),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
