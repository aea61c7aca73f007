"""HIP graph capture and concurrent streams.

The header promises that no call allocates or synchronises, so every call may
be captured into a HIP graph, and that a call's plan (and so its bits)
depends only on its arguments: the few-row split-K takes its exchange buffers
from a workspace (the binding keeps a zero-filled one per stream, made by
torch's allocator; on a fresh stream it is made inside the capture).  The
graph is replayed several times with eager work in between, and every replay
is compared bit for bit with the eager result of the same call."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import quant
from tests.helpers import announce, bf16_bits, dev_f32, dev_sa, dev_u8, quantize_dense

pytestmark = pytest.mark.gpu


def _dense_operands(M, N, K, seed):
    A32, B32 = synth.dense_problem(M, N, K, seed=seed)
    qa, sa, qb, sb = quantize_dense(A32, B32)
    return dev_u8(qa), dev_sa(sa), dev_u8(qb), dev_f32(sb)


def _masked_operands(G, Mc, N, K, seed):
    A32, B32, mask = synth.masked_problem(G, Mc, N, K, seed=seed)
    qs = [quant.quantize_per_token(a) for a in A32.numpy()]
    qa = np.stack([q for q, _ in qs])
    sa = np.stack([s for _, s in qs])
    qbs = [quant.quantize_per_block(b) for b in B32.numpy()]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    return dev_u8(qa), dev_sa(sa, groups=True), dev_u8(qb), dev_f32(sb), torch.from_numpy(mask.astype(np.int32)).cuda()


@pytest.mark.parametrize("fresh_stream", [False, True], ids=["warm-stream", "fresh-stream"])
def test_graph_replays_match_eager(gpu_lib, monkeypatch, fresh_stream):
    """Dense few-row (split K), dense large-tile and masked calls, and the
    power-of-two-factor dense, masked and contiguous calls, captured together.
    On the fresh stream nothing has run before the capture; the captured
    few-row GEMM still takes the split plan of the eager call."""
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("FG_SKINNY", raising=False)
    announce(f"graph capture ({'fresh' if fresh_stream else 'warm'} stream)")
    small = _dense_operands(64, 2112, 7168, seed=1)
    large = _dense_operands(512, 1024, 1024, seed=2)
    masked = _masked_operands(4, 256, 512, 768, seed=3)
    # K tails (K = 1040) on the few-row and large-tile kernels, and the
    # power-of-two-factor GEMM (its 128x256 tile at this shape)
    tail_small = _dense_operands(64, 2112, 1040, seed=4)
    tail_large = _dense_operands(512, 1024, 1040, seed=5)
    gen = torch.Generator(device="cuda").manual_seed(6)
    qa_u, sa_u = gpu_lib.fp8_cast_per_token_ue8m0(torch.randn(512, 1024, device="cuda", generator=gen))
    qb_u, sb_u = gpu_lib.fp8_cast_per_block_ue8m0(torch.randn(4096, 1024, device="cuda", generator=gen))
    # grouped GEMMs with power-of-two factors: masked (the masked problem's
    # counts) and contiguous with a K tail (K = 1040)
    G, Mc, Nm, Km = 4, 256, 512, 768
    kb4 = (Km // 128 + 3) // 4
    qa_m, sa_m = gpu_lib.fp8_cast_per_token_ue8m0(torch.randn(G * Mc, Km, device="cuda", generator=gen))
    sa_m = sa_m.reshape(kb4, G, Mc).permute(1, 0, 2).contiguous()
    qb_m, sb_m = gpu_lib.fp8_cast_per_block_ue8m0(torch.randn(G * Nm, Km, device="cuda", generator=gen))
    masked_u = (qa_m.view(G, Mc, Km), sa_m, qb_m.view(G, Nm, Km), sb_m.view(G, Nm // 128, kb4))
    idx = torch.from_numpy(synth.contiguous_indices([200, 60, 128], pad_to=128)).cuda()
    Mt, Nc, Kc = idx.shape[0], 256, 1040
    qa_c, sa_c = gpu_lib.fp8_cast_per_token_ue8m0(torch.randn(Mt, Kc, device="cuda", generator=gen))
    qb_c, sb_c = gpu_lib.fp8_cast_per_block_ue8m0(torch.randn(3 * Nc, Kc, device="cuda", generator=gen))
    contig_u = (qa_c, sa_c, qb_c.view(3, Nc, Kc), sb_c.view(3, Nc // 128, -1))
    outs = [torch.empty(64, 2112, dtype=torch.bfloat16, device="cuda"),
            torch.empty(512, 1024, dtype=torch.bfloat16, device="cuda"),
            torch.empty(4, 256, 512, dtype=torch.bfloat16, device="cuda"),
            torch.empty(64, 2112, dtype=torch.bfloat16, device="cuda"),
            torch.empty(512, 1024, dtype=torch.bfloat16, device="cuda"),
            torch.empty(512, 4096, dtype=torch.bfloat16, device="cuda"),
            torch.empty(G, Mc, Nm, dtype=torch.bfloat16, device="cuda"),
            torch.empty(Mt, Nc, dtype=torch.bfloat16, device="cuda")]

    def run_all(stream=None):
        gpu_lib.gemm_fp8_nt(*small, outs[0], stream=stream)
        gpu_lib.gemm_fp8_nt(*large, outs[1], stream=stream)
        gpu_lib.gemm_fp8_grouped_masked(*masked[:4], masked[4], outs[2], stream=stream)
        gpu_lib.gemm_fp8_nt(*tail_small, outs[3], stream=stream)
        gpu_lib.gemm_fp8_nt(*tail_large, outs[4], stream=stream)
        gpu_lib.gemm_fp8_nt_ue8m0(qa_u, sa_u, qb_u, sb_u, outs[5], stream=stream)
        gpu_lib.gemm_fp8_grouped_masked_ue8m0(*masked_u, masked[4], outs[6], stream=stream)
        gpu_lib.gemm_fp8_grouped_contiguous_ue8m0(*contig_u, idx, outs[7], stream=stream)

    s = torch.cuda.Stream()
    if not fresh_stream:
        with torch.cuda.stream(s):
            run_all(s)  # creates this stream's workspace
        torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run_all(s)
    torch.cuda.synchronize()

    # eager reference on the default stream (its own workspace), default plan
    for o in outs:
        o.fill_(0)
    run_all()
    torch.cuda.synchronize()
    ref = [bf16_bits(o) for o in outs]
    valid = np.arange(256)[None, :] < masked[4].cpu().numpy()[:, None]
    mapped = idx.cpu().numpy() >= 0

    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bf16_bits(o) for o in outs]
        assert np.array_equal(got[0], ref[0]), rep
        assert np.array_equal(got[1], ref[1]), rep
        assert np.array_equal(got[2][valid], ref[2][valid]), rep
        for i in (3, 4, 5):
            assert np.array_equal(got[i], ref[i]), (rep, i)
        assert np.array_equal(got[6][valid], ref[6][valid]), rep
        assert np.array_equal(got[7][mapped], ref[7][mapped]), rep
        run_all()  # eager work between replays (default plan)
        torch.cuda.synchronize()


def test_concurrent_streams_split_k(gpu_lib, monkeypatch):
    """Two streams run split-K few-row GEMMs at the same time; each has its own
    workspace, so both results equal the sequential ones."""
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.setenv("FG_SKINNY", "1,8")
    announce("concurrent split-K streams")
    ops = [_dense_operands(96, 1000, 4096, seed=10 + i) for i in range(2)]
    seq = []
    for op in ops:
        D = torch.empty(96, 1000, dtype=torch.bfloat16, device="cuda")
        gpu_lib.gemm_fp8_nt(*op, D)
        torch.cuda.synchronize()
        seq.append(bf16_bits(D))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty(96, 1000, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    for _ in range(5):
        for st, op, D in zip(streams, ops, outs):
            with torch.cuda.stream(st):
                for _ in range(3):
                    gpu_lib.gemm_fp8_nt(*op, D, stream=st)
        torch.cuda.synchronize()
        for D, ref in zip(outs, seq):
            assert np.array_equal(bf16_bits(D), ref)


def test_split_plan_does_not_depend_on_capture(gpu_lib, monkeypatch):
    """The decode shape's split plan needs a workspace; the same call made
    eagerly, captured on a fresh stream, and through the C entry point with
    an explicit workspace gives the same bits.  The captured graph is then
    replayed on another stream while eager calls with a different workspace
    run on the capturing one."""
    monkeypatch.delenv("FG_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("FG_SKINNY", raising=False)
    announce("split plan vs capture 64x2112x7168")
    M, N, K = 64, 2112, 7168
    op = _dense_operands(M, N, K, seed=12)
    assert gpu_lib.nt_workspace_bytes(M, N, K) > 0  # the plan splits K
    eager = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    gpu_lib.gemm_fp8_nt(*op, eager)
    torch.cuda.synchronize()
    ref = bf16_bits(eager)
    own = torch.zeros(gpu_lib.nt_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    explicit = torch.empty_like(eager)
    gpu_lib.gemm_fp8_nt(*op, explicit, workspace=own)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(explicit), ref)
    s_cap, s_other = torch.cuda.Stream(), torch.cuda.Stream()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s_cap):
        gpu_lib.gemm_fp8_nt(*op, out, stream=s_cap)
    torch.cuda.synchronize()
    side = torch.empty_like(eager)
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s_other):
            g.replay()
        with torch.cuda.stream(s_cap):
            gpu_lib.gemm_fp8_nt(*op, side, stream=s_cap, workspace=own)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(out), ref), rep
        assert np.array_equal(bf16_bits(side), ref), rep
