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
from tests.gpu_util import check_f32, f32, say

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
