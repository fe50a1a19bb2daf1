"""GPU parity of the grouped (mixture-of-experts) block-scaled GEMM."""

import numpy as np
import pytest
import torch

import workloads
from fp8_fine_grained_amd import binding as fp8
from oracle import gemm, quant
from tests.gpu_util import assert_codes_equal, assert_scales_equal, check_bf16, check_f32, check_guard, f32, guarded, say

pytestmark = pytest.mark.gpu


def _case(offsets, N, K, seed):
    offsets = np.asarray(offsets, dtype=np.int32)
    G = offsets.size - 1
    M = int(offsets[-1])
    x = workloads.dense(seed=seed, M=max(M, 1), N=128, K=K)["x"][:M]
    w = torch.stack([workloads.moe_expert_weight(g, seed=seed, N=N, K=K) for g in range(G)])
    qa, sa = fp8.fp8_quant_act_1x128(x.cuda()) if M else (torch.empty((0, K), dtype=torch.uint8, device="cuda"),
                                                          torch.empty((0, K // 128), device="cuda"))
    qb, sb = fp8.fp8_quant_weight_128x128(w.cuda().view(G * N, K))
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    ra, rsa = quant.quant_1x128(f32(x)) if M else (np.zeros((0, K), np.uint8), np.zeros((0, K // 128), np.float32))
    rb = np.empty((G, N, K), np.uint8)
    rsb = np.empty((G, N // 128, K // 128), np.float32)
    for g in range(G):
        rb[g], rsb[g] = quant.quant_128x128(f32(w[g]))
    assert np.array_equal(qb.cpu().numpy(), rb)
    off = torch.from_numpy(offsets).cuda()
    return (qa, sa, off, qb, sb), (ra, rsa, offsets, rb, rsb)


def _run(g, M, N, dtype, accum):
    buf, y = guarded((M, N), dtype)
    fp8.fp8_block_grouped_gemm(*g, accum=accum, y=y)
    torch.cuda.synchronize()
    check_guard(buf)
    return y


def test_small_ragged_segments():
    sizes = [5, 0, 1, 300, 0, 17, 129, 128]
    off = np.concatenate([[0], np.cumsum(sizes)])
    g, r = _case(off, 256, 512, 11)
    ref = gemm.grouped_gemm(*r)
    say(f"grouped sizes {sizes}, N=256, K=512")
    check_bf16(_run(g, int(off[-1]), 256, torch.bfloat16, "fp8"), ref, "fp8 accum")
    check_f32(_run(g, int(off[-1]), 256, torch.float32, "exact"), ref, "exact accum fp32")


def test_skewed_routing():
    off = workloads.skewed_offsets(3000, 32, 1500, 6)
    g, r = _case(off, 128, 256, 12)
    ref = gemm.grouped_gemm(*r)
    say("grouped skewed: one expert 1500 rows, 6 empty")
    check_bf16(_run(g, 3000, 128, torch.bfloat16, "fp8"), ref, "fp8 accum")


def test_every_live_row_count_of_a_tile():
    """Segments whose last 128-row tile holds 1 .. 128 rows in steps that hit
    every count of live 16-row sub-tiles in both m-parts of the tile (sizes on
    and beside the 16-row boundaries).  Each segment's rows equal, bit for bit,
    the dense kernel on that segment alone (the same 128-K blocks and
    promotion order), and the whole output is within the oracle's bound."""
    sizes = [1, 15, 16, 17, 32, 33, 48, 49, 63, 64, 65, 80, 81, 96, 97, 112, 113, 127, 128, 129, 200, 255, 256, 0, 47]
    off = np.concatenate([[0], np.cumsum(sizes)])
    N, K = 256, 384
    g, r = _case(off, N, K, 41)
    M = int(off[-1])
    say(f"grouped live-row counts: {len(sizes)} segments, {M} rows, N={N}, K={K}")
    y = _run(g, M, N, torch.float32, "fp8")
    qa, sa, _, qb, sb = g
    for e, (lo, hi) in enumerate(zip(off[:-1], off[1:])):
        if hi == lo:
            continue
        yd = fp8.fp8_block_gemm(qa[lo:hi].contiguous(), sa[lo:hi].contiguous(), qb[e].contiguous(),
                                sb[e].contiguous(), accum="fp8", out_dtype=torch.float32)
        assert torch.equal(y[lo:hi], yd), f"segment {e} ({hi - lo} rows) differs from the dense kernel"
    ref = gemm.grouped_gemm(*r)
    check_bf16(_run(g, M, N, torch.bfloat16, "fp8"), ref, "fp8 accum, bf16")
    check_f32(_run(g, M, N, torch.float32, "exact"), ref, "exact accum fp32")


def test_single_group_matches_dense_kernel():
    off = np.array([0, 333])
    g, r = _case(off, 256, 384, 13)
    yg = _run(g, 333, 256, torch.float32, "fp8")
    qa, sa, _, qb, sb = g
    yd = fp8.fp8_block_gemm(qa, sa, qb[0].contiguous(), sb[0].contiguous(), accum="fp8", out_dtype=torch.float32)
    assert torch.equal(yg, yd)


def _gather_case(T, G, topk, N, K, seed):
    """Tokens routed top-k over G experts; the gathered GEMM reads token rows
    through the permutation, the reference reads an explicitly permuted copy."""
    logits = workloads.dense(seed=seed, M=T, N=1, K=G)["x"].float().numpy()
    route = workloads.route_topk(logits, np.zeros(G, np.float32), topk)
    perm, offsets = route[0], route[1]
    x = workloads.dense(seed=seed + 1, M=T, N=128, K=K)["x"]
    w = torch.stack([workloads.moe_expert_weight(g, seed=seed, N=N, K=K) for g in range(G)])
    qt, st = fp8.fp8_quant_act_1x128(x.cuda())
    qb, sb = fp8.fp8_quant_weight_128x128(w.cuda().view(G * N, K))
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    idx = torch.from_numpy(perm.astype(np.int32)).cuda()
    off = torch.from_numpy(offsets).cuda()
    rt, rst = quant.quant_1x128(f32(x))
    assert np.array_equal(qt.cpu().numpy(), rt)
    rb = np.empty((G, N, K), np.uint8)
    rsb = np.empty((G, N // 128, K // 128), np.float32)
    for g in range(G):
        rb[g], rsb[g] = quant.quant_128x128(f32(w[g]))
    ref = gemm.grouped_gemm(rt[perm], rst[perm], offsets, rb, rsb)
    return (qt, st, idx, off, qb, sb), ref, int(offsets[-1])


def test_gather_small():
    g, ref, M = _gather_case(T=97, G=8, topk=3, N=256, K=384, seed=21)
    qt, st, idx, off, qb, sb = g
    say(f"grouped gather: 97 tokens, 8 experts top-3 -> {M} rows, N=256, K=384")
    for accum, dtype in (("fp8", torch.bfloat16), ("exact", torch.float32), ("fp8", torch.float32)):
        buf, y = guarded((M, 256), dtype)
        fp8.fp8_block_grouped_gemm_gather(qt, st, idx, off, qb, sb, accum=accum, y=y)
        torch.cuda.synchronize()
        check_guard(buf)
        if dtype == torch.bfloat16:
            check_bf16(y, ref, "fp8 accum, bf16")
        elif accum == "exact":
            check_f32(y, ref, "exact accum fp32")
        # Gathering only moves the loads: bitwise the same as the grouped GEMM on a permuted copy.
        yp = fp8.fp8_block_grouped_gemm(qt[idx.long()].contiguous(), st[idx.long()].contiguous(), off, qb, sb,
                                        accum=accum, out_dtype=dtype)
        assert torch.equal(y, yp), f"{accum} {dtype}"


def test_expert_parallel_shares_equal_the_full_launch():
    """One GPU's share under expert parallelism is the same gathering launch on a
    contiguous range of experts (their offsets rebased to 0, their weights, the
    index rows routed to them and the matching output rows): eight shares of 8
    of 64 experts reproduce the full launch bit for bit."""
    G, N, K = 64, 256, 512
    g, ref, M = _gather_case(T=512, G=G, topk=8, N=N, K=K, seed=41)
    qt, st, idx, off, qb, sb = g
    say(f"expert-parallel shares: 512 tokens, {G} experts top-8 -> {M} rows, 8 shares of {G // 8}")
    y = fp8.fp8_block_grouped_gemm_gather(qt, st, idx, off, qb, sb, accum="fp8", out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_bf16(y, ref, "full launch")
    off_np = off.cpu().numpy()
    buf, ys = guarded((M, N), torch.bfloat16)
    GS = G // 8
    for e in range(8):
        lo, hi = int(off_np[e * GS]), int(off_np[(e + 1) * GS])
        o = torch.from_numpy((off_np[e * GS:(e + 1) * GS + 1] - lo).astype(np.int32)).cuda()
        fp8.fp8_block_grouped_gemm_gather(qt, st, idx[lo:hi], o, qb[e * GS:(e + 1) * GS], sb[e * GS:(e + 1) * GS],
                                          accum="fp8", y=ys[lo:hi])
    torch.cuda.synchronize()
    check_guard(buf)
    assert torch.equal(ys, y)


def test_gather_repeated_and_unused_tokens():
    # every routed row is token 5 or token 0; most tokens are never read
    T, K, N, G = 40, 256, 256, 3
    x = workloads.dense(seed=31, M=T, N=128, K=K)["x"]
    qt, st = fp8.fp8_quant_act_1x128(x.cuda())
    w = torch.stack([workloads.moe_expert_weight(g, seed=31, N=N, K=K) for g in range(G)])
    qb, sb = fp8.fp8_quant_weight_128x128(w.cuda().view(G * N, K))
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    perm = np.array([5, 0, 5, 5, 0, 5, 0], np.int32)
    offsets = np.array([0, 2, 2, 7], np.int32)
    y = fp8.fp8_block_grouped_gemm_gather(qt, st, torch.from_numpy(perm).cuda(), torch.from_numpy(offsets).cuda(),
                                          qb, sb, accum="exact", out_dtype=torch.float32)
    rt, rst = quant.quant_1x128(f32(x))
    rb = np.stack([quant.quant_128x128(f32(w[g]))[0] for g in range(G)])
    rsb = np.stack([quant.quant_128x128(f32(w[g]))[1] for g in range(G)])
    check_f32(y, gemm.grouped_gemm(rt[perm], rst[perm], offsets, rb, rsb), "repeated tokens, exact")


def test_empty_inputs_are_noops():
    K, N = 256, 128
    a = torch.empty((0, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((0, 2), device="cuda")
    b = torch.zeros((2, N, K), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((2, 1, 2), device="cuda")
    off = torch.zeros(3, dtype=torch.int32, device="cuda")
    y = fp8.fp8_block_grouped_gemm(a, sa, off, b, sb)
    assert y.shape == (0, N)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_full_moe_up_projection():
    """Full MoE size, every output: the routed rows' codes and scales bit-exact
    (the oracle quantises the 8192 tokens; a routed row is its token's row), each
    expert's weight codes and scales bit-exact, and all 65536 x 2048 outputs
    within the bf16 tolerance of the oracle's fp64 grouped GEMM (each expert's
    segment in a spawned worker process, which quantises that expert's weight
    itself)."""
    import hashlib
    import multiprocessing
    import os

    from tests.moe_reference import expert_reference

    say("MoE up-projection: 8192 tokens, 256 experts top-8, W [2048,7168] per expert")
    route = workloads.moe_routing()
    tokens = workloads.moe_tokens()
    perm = torch.from_numpy(route["perm"])
    offsets = route["offsets"]
    say("  generating expert weights")
    w = workloads.moe_expert_weights(range(256))
    say("  quantise + grouped GEMM on GPU")
    xa = tokens.cuda()[perm.cuda()]
    qa, sa = fp8.fp8_quant_act_1x128(xa)
    wd = w.cuda()
    del w
    qb, sb = fp8.fp8_quant_weight_128x128(wd.view(256 * 2048, 7168))
    del wd
    qb, sb = qb.view(256, 2048, 7168), sb.view(256, 16, 56)
    y = fp8.fp8_block_grouped_gemm(qa, sa, torch.from_numpy(offsets).cuda(), qb, sb)
    torch.cuda.synchronize()
    say("  oracle: quantise the tokens")
    rt, rst = quant.quant_1x128(f32(tokens))
    permn = np.asarray(route["perm"])
    assert_codes_equal(qa, rt[permn], "routed row codes")
    assert_scales_equal(sa, rst[permn], "routed row scales")
    jobs = []
    for e in range(256):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            jobs.append((e, rt[permn[lo:hi]], rst[permn[lo:hi]]))
    nproc = max(1, min(16, len(os.sched_getaffinity(0))))
    say(f"  oracle: {len(jobs)} experts in {nproc} worker processes, all {int(offsets[-1])} rows")
    ref = np.zeros((int(offsets[-1]), 2048))
    done = 0
    with multiprocessing.get_context("spawn").Pool(nproc) as pool:
        for e, code_hash, scale_hash, ref_rows in pool.imap_unordered(expert_reference, jobs):
            assert hashlib.sha256(qb[e].cpu().numpy().tobytes()).hexdigest() == code_hash, f"expert {e} codes"
            assert hashlib.sha256(sb[e].cpu().numpy().tobytes()).hexdigest() == scale_hash, f"expert {e} scales"
            ref[int(offsets[e]):int(offsets[e + 1])] = ref_rows
            done += 1
            if done % 32 == 0:
                say(f"  oracle: {done} of {len(jobs)} experts done")
    check_bf16(y, ref, f"all {int(offsets[-1])} routed rows x 2048")
    say("  FP8 dispatch by index: quantise the 8192 tokens, gather rows inside the GEMM")
    qt, st = fp8.fp8_quant_act_1x128(tokens.cuda())
    idx = perm.to(torch.int32).cuda()
    assert torch.equal(qt[idx.long()], qa) and torch.equal(st[idx.long()], sa)
    yg = fp8.fp8_block_grouped_gemm_gather(qt, st, idx, torch.from_numpy(offsets).cuda(), qb, sb)
    assert torch.equal(yg, y)
