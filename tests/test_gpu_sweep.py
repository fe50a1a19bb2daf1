"""Seeded randomized parity sweep: random shapes through every GEMM mode of the
library (dense and grouped, gathering, block- and row-scaled weights, FP8,
exact and scaled accumulation, bf16 and fp32 outputs), each compared element
by element with the oracle.  The shapes cover every tile family the library
dispatches to: N a multiple of 256, of 896 (224-wide tiles) and an odd
multiple of 128 (the 128 x 128 kernel), ragged M, K from one to sixteen blocks,
and segment layouts with empty and one-row experts."""

import numpy as np
import pytest
import torch

import workloads
from fp8_fine_grained_amd import binding as fp8
from oracle import gemm, quant
from tests.gpu_util import check_bf16, check_f32, check_guard, f32, fp8_mfma_bound_separable, guarded, say

pytestmark = pytest.mark.gpu


def _dense_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        family = ["n256", "n896", "n128odd"][i % 3]
        N = {"n256": 256 * int(rng.integers(1, 5)), "n896": 896 * int(rng.integers(1, 3)),
             "n128odd": 128 * (2 * int(rng.integers(0, 4)) + 1)}[family]
        M = int(rng.integers(1, 700))
        K = 128 * int(rng.integers(1, 17))
        mode = "row" if rng.random() < 0.3 else "block"
        accums = ["fp8", "exact"] + (["scaled"] if mode == "block" and family != "n128odd" else [])
        accum = accums[int(rng.integers(0, len(accums)))]
        out = "fp32" if rng.random() < 0.5 else "bf16"
        cases.append((i, M, N, K, mode, accum, out))
    return cases


def _check(y, ref, qa, sa, qb, sb, mode, accum, out, what):
    if out == "bf16":
        check_bf16(y, ref, what)
    elif accum == "exact":
        check_f32(y, ref, what)
    else:
        g = f32(y).astype(np.float64)
        bound = fp8_mfma_bound_separable(qa, sa, qb, sb, mode)
        err = np.abs(g - ref)
        say(f"  {what}: max err/bound {np.max(err / bound):.3f}")
        assert np.all(np.isfinite(g)) and np.all(err <= bound), what


@pytest.mark.parametrize("case", _dense_cases(24, 2024), ids=lambda c: "dense{}_{}x{}x{}_{}_{}_{}".format(*c))
def test_dense_sweep(case):
    i, M, N, K, mode, accum, out = case
    pow2 = accum == "scaled"
    d = workloads.dense(seed=100 + i, M=M, N=N, K=K)
    x, w = d["x"], d["w"]
    qa, sa = fp8.fp8_quant_act_1x128(x.cuda(), pow2=pow2)
    scale = "pow2" if pow2 else "amax"
    ra, rsa = quant.quant_1x128(f32(x), scale=scale)
    if mode == "row":
        qb, sb = fp8.fp8_quant_act_1x128(w.cuda(), pow2=pow2)
        rb, rsb = quant.quant_1x128(f32(w), scale=scale)
    else:
        qb, sb = fp8.fp8_quant_weight_128x128(w.cuda(), pow2=pow2)
        rb, rsb = quant.quant_128x128(f32(w), scale=scale)
    assert np.array_equal(qa.cpu().numpy(), ra) and np.array_equal(qb.cpu().numpy(), rb)
    buf, y = guarded((M, N), torch.float32 if out == "fp32" else torch.bfloat16)
    fp8.fp8_block_gemm(qa, sa, qb, sb, b_scale_mode=mode, accum=accum, y=y)
    torch.cuda.synchronize()
    check_guard(buf)
    ref = gemm.block_gemm(ra, rsa, rb, rsb, mode=mode)
    _check(y, ref, ra, rsa, rb, rsb, mode, accum, out, f"{M}x{N}x{K} {mode} {accum} {out}")


def _grouped_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        G = int(rng.integers(1, 13))
        sizes = rng.integers(0, 400, G)
        sizes[rng.random(G) < 0.2] = 0
        sizes[rng.random(G) < 0.1] = 1
        N = 256 * int(rng.integers(1, 4)) if i % 4 else 128 * (2 * int(rng.integers(0, 3)) + 1)
        K = 128 * int(rng.integers(1, 13))
        accums = ["fp8", "exact"] + (["scaled"] if N % 256 == 0 else [])
        accum = accums[int(rng.integers(0, len(accums)))]
        out = "fp32" if rng.random() < 0.5 else "bf16"
        gather = bool(N % 256 == 0 and rng.random() < 0.5)
        cases.append((i, tuple(int(s) for s in sizes), N, K, accum, out, gather))
    return cases


@pytest.mark.parametrize("case", _grouped_cases(16, 2025),
                         ids=lambda c: "grouped{}_G{}_N{}_K{}_{}_{}_{}".format(c[0], len(c[1]), *c[2:6],
                                                                                 "gather" if c[6] else "rows"))
def test_grouped_sweep(case):
    i, sizes, N, K, accum, out, gather = case
    pow2 = accum == "scaled"
    scale = "pow2" if pow2 else "amax"
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offsets[-1])
    rng = np.random.default_rng(300 + i)
    w = torch.stack([workloads.moe_expert_weight(g, seed=200 + i, N=N, K=K) for g in range(G)])
    qb, sb = fp8.fp8_quant_weight_128x128(w.cuda().view(G * N, K), pow2=pow2)
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    # the routed rows: token rows by index (with repeats and unused tokens) when gathering
    T = max(1, M // 2 + 1)
    tokens = workloads.dense(seed=400 + i, M=T, N=128, K=K)["x"]
    idx = rng.integers(0, T, M).astype(np.int32)
    rt, rst = quant.quant_1x128(f32(tokens), scale=scale)
    ra, rsa = rt[idx], rst[idx]
    say(f"grouped sizes {list(sizes)}, N={N}, K={K}, {accum}, {out}, {'gather' if gather else 'rows'}")
    buf, y = guarded((M, N), torch.float32 if out == "fp32" else torch.bfloat16)
    off = torch.from_numpy(offsets).cuda()
    if gather:
        qt, st = fp8.fp8_quant_act_1x128(tokens.cuda(), pow2=pow2)
        assert np.array_equal(qt.cpu().numpy(), rt)
        fp8.fp8_block_grouped_gemm_gather(qt, st, torch.from_numpy(idx).cuda(), off, qb, sb, accum=accum, y=y)
    else:
        qa, sa = fp8.fp8_quant_act_1x128(tokens[torch.from_numpy(idx).long()].cuda(), pow2=pow2) if M else (
            torch.empty((0, K), dtype=torch.uint8, device="cuda"), torch.empty((0, K // 128), device="cuda"))
        fp8.fp8_block_grouped_gemm(qa, sa, off, qb, sb, accum=accum, y=y)
    torch.cuda.synchronize()
    check_guard(buf)
    if M == 0:
        return
    ref = np.zeros((M, N))
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            rb, rsb = quant.quant_128x128(f32(w[g]), scale=scale)
            assert np.array_equal(qb[g].cpu().numpy(), rb)
            ref[lo:hi] = gemm.block_gemm(ra[lo:hi], rsa[lo:hi], rb, rsb)
            yg = y[lo:hi]
            _check(yg, ref[lo:hi], ra[lo:hi], rsa[lo:hi], rb, rsb, "block", accum, out,
                   f"expert {g} rows {lo}..{hi}")
