"""Benchmark of the FP8 fine-grained-scaled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: the dense inference GEMMs at M=4096 with (N, K) in
{(2112,7168), (24576,1536), (7168,16384), (4096,7168), (7168,2048)}.
Inputs are seeded synthetic N(0,1) fp32 matrices (``synth``), cast to e4m3
with the library's own per-token / per-block cast kernels and kept resident in
HBM; a *step* is one pass over every GEMM of the workload (the activation cast
is timed separately and reported under ``cast``).  Every GEMM launch is timed
with HIP events on the stream it is launched on.

One JSON line is printed with the aggregate throughput (TFLOPS = total
algorithmic flops / total GEMM time), per-shape TFLOPS / GB/s / roofline
fractions, a ``roofline`` object for the GEMM kernel (MFMA-bound, against the
published 5.0 PFLOP/s dense FP8 peak; ``traffic`` is the HBM bytes per launch
measured with rocprofv3 counters when the committed counter summary matches
the current kernel sources, else null) and a ``cpu_baseline`` object: the CPU
oracle timed on a bounded sample of output blocks of the same workload.
``other_configs`` adds per-shape figures for the small-M dense, contiguous
and masked workloads; for the dense M=4096 shapes, the contiguous GEMM and
the masked decode with power-of-two (UE8M0) factors on the scaled MFMA; for
the dense shapes with an fp32 addend (D = C + A B^T) and in the NN and TN
storage layouts, each timed beside the plain GEMM; and for the K-grouped TN
GEMM of weight gradients.
Skip them with --no-other-configs.
"""

from __future__ import annotations

import argparse
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
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_dense_m4096_traffic.json")


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


def dense_bytes(M, N, K) -> int:
    """Algorithmic HBM bytes of one dense GEMM: A, B once, scales, D once."""
    Kb, Nb = K // 128, -(-N // 128)
    return M * K + N * K + 4 * (M * Kb + Nb * Kb) + 2 * M * N


class Problem:
    """One resident dense problem: fp32 source -> device casts -> e4m3 operands."""

    def __init__(self, M, N, K, seed=0):
        self.M, self.N, self.K = M, N, K
        A32, B32 = synth.dense_problem(M, N, K, seed=seed)
        self.A32_cpu, self.B32_cpu = A32, B32
        self.a32 = A32.cuda()
        self.qa, self.sa = fg.fp8_cast_per_token(self.a32)
        b32 = B32.cuda()
        self.qb, self.sb = fg.fp8_cast_per_block(b32)
        del b32
        self.D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        self.flops = 2 * M * N * K
        self.bytes = dense_bytes(M, N, K)

    def run(self, stream):
        fg.gemm_fp8_nt(self.qa, self.sa, self.qb, self.sb, self.D, stream=stream)

    def cast(self, stream):
        fg.fp8_cast_per_token(self.a32, self.qa, self.sa, stream=stream)


def time_steps(problems, steps, warmup):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for pb in problems:
            pb.run(stream)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in problems]
          for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        for i, pb in enumerate(problems):
            ev[s][i][0].record(stream)
            pb.run(stream)
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[a.elapsed_time(b) for (a, b) in row] for row in ev])  # ms [steps, shapes]
    return wall, per


def time_casts(problems):
    """Activation-cast time per problem: GPU time per launch from graph
    replay, so that a short cast is not charged the host's submit time."""
    out = []
    for pb in problems:
        ms = graph_time(lambda i, pb=pb: pb.cast(torch.cuda.current_stream()))
        nbytes = pb.M * pb.K * 5 + 4 * pb.M * (pb.K // 128)
        out.append({"M": pb.M, "K": pb.K, "us": round(ms * 1e3, 2), "gbs": round(nbytes / ms / 1e6, 1),
                    "pct_hbm": round(nbytes / ms / 1e6 / PEAK_HBM_GBS * 100, 1)})
    return out


def graph_time(launch, launches: int = 20, reps: int = 5) -> float:
    """GPU milliseconds per launch of `launch(i)` without host overhead: the
    launches are captured into one HIP graph (after warm-up calls on the same
    stream, which also create any workspace) and the graph is replayed."""
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
    """Median GPU milliseconds of `launch()` over `reps` event-timed calls,
    after three untimed ones."""
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


def other_configs():
    """Per-shape throughput of the small-M dense, contiguous and masked
    workloads.  Weight operands are rotated over copies totalling more than
    the 256 MB last-level cache, so every launch reads them from HBM; the
    memory-bound launches are timed by graph replay (their GPU time is a few
    microseconds, below the host's per-call cost)."""
    out = []
    # the small dense problem 128x256x512: a launch-latency case, timed by
    # graph replay like the memory-bound launches
    for (M, N, K) in synth.SMALL_DENSE.shapes:
        A32, B32 = synth.dense_problem(M, N, K, seed=0)
        qa, sa = fg.fp8_cast_per_token(A32.cuda())
        qb, sb = fg.fp8_cast_per_block(B32.cuda())
        D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ms = graph_time(lambda i: fg.gemm_fp8_nt(qa, sa, qb, sb, D))
        out.append(shape_entry("dense_small", (M, N, K), ms, 2 * M * N * K, dense_bytes(M, N, K), "launch"))
        progress(f"small dense {M}x{N}x{K}: {ms * 1e3:.2f} us")
    for (M, N, K) in synth.DENSE_SMALL_M.shapes:
        A32, B32 = synth.dense_problem(M, N, K, seed=0)
        qa, sa = fg.fp8_cast_per_token(A32.cuda())
        qb, sb = fg.fp8_cast_per_block(B32.cuda())
        copies = [qb] + [qb.clone() for _ in range(max(1, int(600e6 // (N * K))))]
        D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ms = graph_time(lambda i: fg.gemm_fp8_nt(qa, sa, copies[i % len(copies)], sb, D))
        Kb = K // 128
        nbytes = M * K + N * K + 4 * (M * Kb + -(-N // 128) * Kb) + 2 * M * N
        out.append(shape_entry("dense_small_m", (M, N, K), ms, 2 * M * N * K, nbytes, "hbm"))
        del copies
        progress(f"small-M dense {M}x{N}x{K}: {ms * 1e3:.2f} us")
    # the dense M=4096 shapes with power-of-two (UE8M0) factors (GPU casts)
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
    # the dense M=4096 shapes with an fp32 addend, D = C + A B^T; the plain
    # GEMM on the same operands is timed beside it
    for (M, N, K) in synth.DENSE_M4096.shapes:
        A32, B32 = synth.dense_problem(M, N, K, seed=0)
        qa, sa = fg.fp8_cast_per_token(A32.cuda())
        qb, sb = fg.fp8_cast_per_block(B32.cuda())
        del A32, B32
        C = torch.randn(M, N, generator=torch.Generator().manual_seed(1)).cuda()
        D = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ms = event_time(lambda: fg.gemm_fp8_nt_c(qa, sa, qb, sb, C, D))
        plain = event_time(lambda: fg.gemm_fp8_nt(qa, sa, qb, sb, D))
        Kb = K // 128
        nbytes = M * K + N * K + 4 * (M * Kb + -(-N // 128) * Kb) + 4 * M * N + 2 * M * N
        e = shape_entry("dense_m4096_addend", (M, N, K), ms, 2 * M * N * K, nbytes, "mfma")
        e["plain_us"] = round(plain * 1e3, 2)
        out.append(e)
        # the NN and TN storage layouts (transposes into the workspace + the
        # NT GEMM); bytes count the operands once, as stored
        for layout in ("nn", "tn"):
            As = qa.t().contiguous() if layout[0] == "t" else qa
            Bs = qb.t().contiguous() if layout[1] == "n" else qb
            ws = torch.empty(fg.layout_workspace_bytes(layout, M, N, K), dtype=torch.uint8, device="cuda")
            gemm = getattr(fg, "gemm_fp8_" + layout)
            ms = event_time(lambda: gemm(As, sa, Bs, sb, D, workspace=ws))
            nbytes = M * K + N * K + 4 * (M * Kb + -(-N // 128) * Kb) + 2 * M * N
            e = shape_entry("dense_m4096_" + layout, (M, N, K), ms, 2 * M * N * K, nbytes, "mfma")
            e["plain_us"] = round(plain * 1e3, 2)
            out.append(e)
            del As, Bs, ws
        del qa, qb, C, D
        progress(f"addend and layouts {M}x{N}x{K} done")
    # K-grouped TN (weight gradients of the contiguous workload: 8 experts x
    # 4096 tokens, M = 4096, N = 7168); operands drawn on the GPU from a
    # seeded generator and cast there
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
    e = shape_entry("k_grouped_tn_8x4096", (len(ks), M, N, ks[0]), ms, 2 * M * N * Kt, nbytes, "mfma")
    out.append(e)
    del As, Bs, D, ws
    progress(f"K-grouped TN: {ms * 1e3:.2f} us")
    G, rows, N, K = synth.CONTIGUOUS_8x4096.shapes[0]
    A32, B32, idx = synth.contiguous_problem([rows] * G, N, K, seed=0)
    qa, sa = fg.fp8_cast_per_token(A32.cuda())
    qb, sb = fg.fp8_cast_per_block(B32.reshape(G * N, K).cuda())
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    mi = torch.from_numpy(idx.astype(np.int32)).cuda()
    D = torch.empty(idx.shape[0], N, dtype=torch.bfloat16, device="cuda")
    fg.gemm_fp8_grouped_contiguous(qa, sa, qb, sb, mi, D)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fg.gemm_fp8_grouped_contiguous(qa, sa, qb, sb, mi, D)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    Mt = idx.shape[0]
    out.append(shape_entry("contiguous_8x4096", (G, rows, N, K), float(np.median(ts)), 2 * Mt * N * K,
                           Mt * K + G * N * K + 2 * Mt * N, "mfma"))
    del qa, qb
    # the same GEMM with power-of-two (UE8M0) factors
    qa, sa = fg.fp8_cast_per_token_ue8m0(A32.cuda())
    qb, sb = fg.fp8_cast_per_block_ue8m0(B32.reshape(G * N, K).cuda())
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, -1)
    ms = event_time(lambda: fg.gemm_fp8_grouped_contiguous_ue8m0(qa, sa, qb, sb, mi, D), reps=5)
    out.append(shape_entry("contiguous_8x4096_ue8m0", (G, rows, N, K), ms, 2 * Mt * N * K,
                           Mt * K + G * N * K + 2 * Mt * N, "mfma"))
    del A32, B32, qa, qb, D
    progress("contiguous done")
    for (G, Mc, N, K) in synth.MASKED_16x256.shapes:
        A32, B32, mask = synth.masked_problem(G, Mc, N, K, seed=0)
        qa = torch.empty(G, Mc, K, dtype=torch.uint8, device="cuda")
        sa = fg.empty_activation_scales(Mc, K, groups=G)
        for g in range(G):
            fg.fp8_cast_per_token(A32[g].cuda(), qa[g], sa[g])
        qb, sb = fg.fp8_cast_per_block(B32.reshape(G * N, K).cuda())
        qb, sb = qb.view(G, N, K), sb.view(G, -(-N // 128), K // 128)
        copies = [qb] + [qb.clone() for _ in range(max(1, int(700e6 // (G * N * K))))]
        mt = torch.from_numpy(np.asarray(mask, np.int32)).cuda()
        D = torch.empty(G, Mc, N, dtype=torch.bfloat16, device="cuda")
        em = int(np.mean(mask))
        ms = graph_time(lambda i: fg.gemm_fp8_grouped_masked(qa, sa, copies[i % len(copies)], sb, mt, D, expected_m=em),
                        launches=10)
        rv = int(np.sum(mask))
        out.append(shape_entry("masked_16x256", (G, Mc, N, K), ms, 2 * rv * N * K, rv * K + G * N * K + 2 * rv * N,
                               "hbm"))
        del copies, qa, qb
        progress(f"masked {G}x{Mc}x{N}x{K}: {ms * 1e3:.2f} us")
        # the same decode step with power-of-two (UE8M0) factors
        kb4 = (K // 128 + 3) // 4
        qa = torch.empty(G, Mc, K, dtype=torch.uint8, device="cuda")
        sa = torch.empty(G, kb4, fg.aligned_scale_ld(Mc), dtype=torch.int32, device="cuda")[:, :, :Mc]
        for g in range(G):
            fg.fp8_cast_per_token_ue8m0(A32[g].cuda(), qa[g], sa[g])
        qb, sb = fg.fp8_cast_per_block_ue8m0(B32.reshape(G * N, K).cuda())
        qb, sb = qb.view(G, N, K), sb.view(G, -(-N // 128), kb4)
        copies = [qb] + [qb.clone() for _ in range(max(1, int(700e6 // (G * N * K))))]
        ms = graph_time(lambda i: fg.gemm_fp8_grouped_masked_ue8m0(qa, sa, copies[i % len(copies)], sb, mt, D),
                        launches=10)
        out.append(shape_entry("masked_16x256_ue8m0", (G, Mc, N, K), ms, 2 * rv * N * K,
                               rv * K + G * N * K + 2 * rv * N, "hbm"))
        del copies, qa, qb, D
        progress(f"masked ue8m0 {G}x{Mc}x{N}x{K}: {ms * 1e3:.2f} us")
    return out


def cpu_baseline(problems, budget_s: float = 15.0):
    """The CPU oracle (fp64 blockwise GEMM) on a bounded sample of output
    blocks of every shape: rows [0, ms) x columns [0, ns) at full K, with the
    sample operands quantised by the oracle's own quantiser."""
    from oracle import gemm as ogemm, quant

    try:
        from threadpoolctl import threadpool_info

        cores = max([t.get("num_threads", 0) for t in threadpool_info() if t.get("user_api") == "blas"] or [0])
    except Exception:  # pragma: no cover
        cores = 0
    cores = cores or len(os.sched_getaffinity(0))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info

        blas = ", ".join(sorted({f"{t.get('internal_api')} {t.get('version')}" for t in threadpool_info()
                                 if t.get("user_api") == "blas"}))
    except Exception:  # pragma: no cover
        blas = ""
    # calibrate on the first shape, then size the sample to the budget
    ms, ns = 64, 256
    samples = []
    for pb in problems:
        qa, sa = quant.quantize_per_token(pb.A32_cpu[:ms].numpy())
        qb, sb = quant.quantize_per_block(pb.B32_cpu[:ns].numpy())
        samples.append((qa, sa, qb, sb, pb.K))
    t0 = time.perf_counter()
    flops = 0
    for qa, sa, qb, sb, K in samples:
        ogemm.gemm_nt(qa, sa, qb, sb)
        flops += 2 * ms * ns * K
    dt = time.perf_counter() - t0
    reps = max(1, int(budget_s / max(dt, 1e-3)))
    t0 = time.perf_counter()
    for _ in range(reps):
        for qa, sa, qb, sb, K in samples:
            ogemm.gemm_nt(qa, sa, qb, sb)
    dt = time.perf_counter() - t0
    return {
        "value": round(flops * reps / dt / 1e12, 6),
        "unit": "TFLOPS",
        "cores": int(cores),
        "kind": "oracle",
        "cpu_model": cpu_model,
        "blas": blas,
        "sample": f"fp64 blockwise oracle on D[0:{ms}, 0:{ns}] at full K of each of the {len(problems)} shapes, "
                  f"{reps} passes, {dt:.1f} s",
    }


def traffic_per_launch():
    """HBM bytes per GEMM launch from the committed counter summary, if it
    was taken on the current kernel sources."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            summ = json.load(f)
    except OSError:
        return None
    if summ.get("kernel_source_hash") != kernel_source_hash():
        return None
    return summ.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_m4096", choices=["dense_m4096", "dense_small_m"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the small-M dense, contiguous and masked per-shape measurements")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 3 times (counter calibration)")
    args = ap.parse_args()
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
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    fg.load_library()
    wl = synth.WORKLOADS[args.workload]
    problems = [Problem(*s, seed=0) for s in wl.shapes]
    torch.cuda.synchronize()

    progress(f"{len(problems)} problems resident")
    wall, per = time_steps(problems, args.steps, args.warmup)
    progress(f"{args.steps} timed steps: {wall / args.steps * 1e3:.3f} ms per step")
    casts = time_casts(problems)
    others = None if args.no_other_configs else other_configs()
    gemm_ms = per.sum(axis=1)  # GEMM time per step (sum of launch durations)
    total_flops = sum(pb.flops for pb in problems)
    total_bytes = sum(pb.bytes for pb in problems)
    step_ms = float(np.mean(gemm_ms))
    value = total_flops / (step_ms * 1e-3) / 1e12
    shapes = []
    for i, pb in enumerate(problems):
        ms = float(np.mean(per[:, i]))
        tf = pb.flops / ms / 1e9
        gbs = pb.bytes / ms / 1e6
        shapes.append({"M": pb.M, "N": pb.N, "K": pb.K, "us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                       "pct_mfma": round(tf / PEAK_FP8_TFLOPS * 100, 1), "gbs": round(gbs, 1),
                       "pct_hbm": round(gbs / PEAK_HBM_GBS * 100, 1)})
    achieved = total_flops / (float(np.sum(per)) / args.steps * 1e-3) / 1e12  # flops / mean launch time, aggregated
    launches = len(problems)
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
        "config": {"workload": wl.name, "shapes": [list(s) for s in wl.shapes], "gemm_ms_per_step": round(step_ms, 4),
                   "gbs": round(total_bytes / (step_ms * 1e-3) / 1e9, 1)},
        "shapes": shapes,
        "cast": casts,
        "other_configs": others,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic_per_launch(),
            "kernel": "gemm_fp8_big_kernel (dense)",
            "flops_per_launch": total_flops / launches,
            "launch_us": round(float(np.sum(per)) / args.steps / launches * 1e3, 2),
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(problems),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
