"""HIP graph capture of a whole quantise + GEMM step (the small case).

The library's entry points only enqueue kernels on the caller's stream (no
allocation, no host synchronisation, no memset nodes), so a step can be
captured once and replayed.  Each replay is checked bit for bit against the
eager result, with the program's own eager work and synchronisations between
the replays, and the eager result against the oracle.
"""

import numpy as np
import pytest
import torch

import workloads
from fp8_fine_grained_amd import binding as fp8
from oracle import gemm, quant
from tests.gpu_util import check_bf16, check_f32, f32, say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    t = workloads.tiny()
    x, w = t["x"].cuda(), t["w"].cuda()
    M, K = x.shape
    N = w.shape[0]
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step():
        fp8.fp8_quant_act_1x128(x, qa, sa)
        fp8.fp8_quant_weight_128x128(w, qb, sb)
        fp8.fp8_block_gemm(qa, sa, qb, sb, accum="exact", y=y)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (qa, sa, qb, sb, y)]
    ra, rsa = quant.quant_1x128(f32(t["x"]))
    rb, rsb = quant.quant_128x128(f32(t["w"]))
    assert np.array_equal(eager[0].cpu().numpy(), ra) and np.array_equal(eager[2].cpu().numpy(), rb)
    check_f32(eager[4], gemm.block_gemm(ra, rsa, rb, rsb), "eager step")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"replay {rep}")
        for t_ in (qa, sa, qb, sb, y):
            t_.zero_()  # eager work between replays: the replay must rewrite every output
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((qa, sa, qb, sb, y), eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep} differs"


def test_graph_dense_step_and_k_split_replays():
    """The dense projection step at its full size (one-launch X + W quantiser,
    FP8 GEMM with bf16 output) and an fp32 GEMM whose partial last round runs as
    K-split parts (zero-fill kernel plus fp32 atomic adds), captured in one graph.
    The bf16 step replays bit for bit; the K-split output's split tiles add their
    parts in completion order, so each replay matches the eager result to the
    last bits of those sums (and exactly everywhere else)."""
    d = workloads.dense()
    x, w = d["x"].cuda(), d["w"].cuda()
    M, K = x.shape
    N = w.shape[0]
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    # 4352 x 4096 x 1024 in exact mode: 544 tiles of 128 x 256, the last 32 in 8 K parts each
    s = workloads.dense(M=4352, N=4096, K=1024)
    qs, ss = fp8.fp8_quant_act_1x128(s["x"].cuda())
    qv, sv = fp8.fp8_quant_weight_128x128(s["w"].cuda())
    ys = torch.empty((4352, 4096), dtype=torch.float32, device="cuda")

    def step():
        fp8.fp8_quant_act_weight(x, w, qa, sa, qb, sb)
        fp8.fp8_block_gemm(qa, sa, qb, sb, y=y)
        fp8.fp8_block_gemm(qs, ss, qv, sv, accum="exact", y=ys)

    say("dense step + K-split fp32 GEMM, eager")
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (qa, sa, qb, sb, y, ys)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    outs = (qa, sa, qb, sb, y, ys)
    for rep in range(4):
        say(f"replay {rep}")
        for t_ in outs:
            t_.fill_(7)  # eager work between replays: the replay must rewrite every output
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs[:5], eager[:5]):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep} differs"
        diff = (ys - eager[5]).abs()
        assert torch.all(diff <= 1e-6 * eager[5].abs() + 1e-7 * float(eager[5].abs().max())), \
            f"replay {rep}: K-split output differs beyond the addition order"
        same = float((diff == 0).float().mean())
        say(f"  K-split output: {100 * same:.1f}% of elements bit-identical")
        assert same >= 0.9  # only the 32 split tiles (32 of 544) may differ


def test_graph_moe_gather_step_replays():
    """An MoE step (1x128 quantisation of the tokens, then the grouped GEMM that
    reads each routed row from its token by index, segment offsets on the
    device) captured in a graph: no host synchronisation, so every replay
    equals the eager step bit for bit, after eager writes to its outputs, and
    the eager result equals the oracle's per-expert GEMMs within the bf16 bound."""
    T, E, topk, N, K = 512, 16, 4, 256, 512
    route = workloads.moe_routing(seed=9, T=T, E=E, topk=topk)
    tokens = workloads.moe_tokens(seed=9, T=T, H=K).cuda()
    w = torch.stack([workloads.moe_expert_weight(g, seed=9, N=N, K=K) for g in range(E)]).cuda()
    qb, sb = fp8.fp8_quant_weight_128x128(w.view(E * N, K))
    qb, sb = qb.view(E, N, K), sb.view(E, N // 128, K // 128)
    idx = torch.from_numpy(route["perm"].astype(np.int32)).cuda()
    off = torch.from_numpy(route["offsets"]).cuda()
    qt = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    st = torch.empty((T, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((idx.numel(), N), dtype=torch.bfloat16, device="cuda")

    def step():
        fp8.fp8_quant_act_1x128(tokens, qt, st)
        fp8.fp8_block_grouped_gemm_gather(qt, st, idx, off, qb, sb, accum="fp8", y=y)

    say(f"MoE gather step {T} tokens, {E} experts top-{topk}, eager")
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (qt, st, y)]
    rt, rst = quant.quant_1x128(f32(tokens))
    assert np.array_equal(eager[0].cpu().numpy(), rt)
    offsets = route["offsets"]
    perm = route["perm"]
    ref = np.zeros((idx.numel(), N))
    for g in range(E):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            rb, rsb = quant.quant_128x128(f32(w[g]))
            ref[lo:hi] = gemm.block_gemm(rt[perm[lo:hi]], rst[perm[lo:hi]], rb, rsb)
    check_bf16(eager[2], ref, "eager MoE step")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"replay {rep}")
        for t_ in (qt, st, y):
            t_.fill_(3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((qt, st, y), eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep} differs"


def test_two_streams_run_independent_steps():
    """The library keeps no device state between calls (no scratch buffer, no
    counters): two steps enqueued on two streams at once, each with its own
    outputs, give the same results as the steps run one after the other."""
    a = workloads.dense(seed=21, M=640, N=512, K=1024)
    b = workloads.dense(seed=22, M=384, N=768, K=512)
    ops = []
    for d in (a, b):
        x, w = d["x"].cuda(), d["w"].cuda()
        ops.append((x, w))
    seq = []
    for x, w in ops:
        qa, sa, qb, sb = fp8.fp8_quant_act_weight(x, w)
        seq.append((qa, sa, qb, sb, fp8.fp8_block_gemm(qa, sa, qb, sb, accum="exact", out_dtype=torch.float32)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    par = [None, None]
    for rep in range(3):
        for i, ((x, w), s) in enumerate(zip(ops, streams)):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                qa, sa, qb, sb = fp8.fp8_quant_act_weight(x, w, stream=s)
                y = fp8.fp8_block_gemm(qa, sa, qb, sb, accum="exact", out_dtype=torch.float32, stream=s)
                par[i] = (qa, sa, qb, sb, y)
        torch.cuda.synchronize()
        for i in range(2):
            for got, want in zip(par[i], seq[i]):
                assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"stream {i}, round {rep}"
    say("two streams: both steps equal to the sequential results, three rounds")
