"""GPU parity of the power-of-two (E8M0) scale path against the oracle.

Quantisers: codes and scales bit-exact against oracle.quant with scale="pow2".
GEMM with the scales applied by the matrix cores (accum="scaled"): the products
of a K block are summed like the FP8 matrix-core mode, so fp32 outputs are held
to the same derived per-element bound (tests.gpu_util.fp8_mfma_bound), and
bf16 outputs to half a bf16 ulp + 8e-3 * rms(ref).
"""

import numpy as np
import pytest
import torch

import workloads
from fp8_fine_grained_amd import binding as fp8
from oracle import gemm, quant
from tests.gpu_util import (assert_codes_equal, assert_scales_equal, check_bf16, check_guard, f32,
                            fp8_mfma_bound, fp8_mfma_bound_separable, frob_rel, guarded, say)
from tests.test_gpu_quant import _special_tiles

pytestmark = pytest.mark.gpu


def _act(x_cpu, what, transposed=False):
    """x_cpu [M, K] (or physical [T, C] read along T when transposed)."""
    say(f"pow2 quant_act {'transposed ' if transposed else ''}{what} {tuple(x_cpu.shape)} {x_cpu.dtype}")
    x = x_cpu.cuda()
    src = x.t() if transposed else x
    M, K = src.shape
    qb, q = guarded((M, K), torch.uint8)
    sbuf, s = guarded((M, K // 128), torch.float32)
    fp8.fp8_quant_act_1x128(src, q, s, pow2=True)
    torch.cuda.synchronize()
    check_guard(qb)
    check_guard(sbuf)
    ref = f32(x_cpu).T.copy() if transposed else f32(x_cpu)
    q_ref, s_ref = quant.quant_1x128(ref, scale="pow2")
    assert_codes_equal(q, q_ref, what)
    assert_scales_equal(s, s_ref, what)
    return q, s


def test_act_rows_and_special_tiles():
    _act(workloads.quant_act(M=517, K=7168), "student-t")
    _act(workloads.dense(M=300, N=128, K=1024)["x"], "dense-like ragged")
    x = _special_tiles()
    _act(torch.from_numpy(x), "special fp32")
    _act(workloads.to_bf16(x), "special bf16")


def test_act_transposed():
    d = workloads.wgrad(T=384, C=200, Cin=136)
    _act(d["dy"], "dY", transposed=True)
    _act(torch.from_numpy(_special_tiles().T.copy()), "special fp32", transposed=True)


def test_weight():
    for w, what in ((workloads.tiny()["w"], "tiny fp32"),
                    (workloads.dense(M=128, N=384, K=640)["w"], "dense-like bf16")):
        say(f"pow2 quant_weight {what} {tuple(w.shape)}")
        N, K = w.shape
        qb, q = guarded((N, K), torch.uint8)
        sbuf, s = guarded((N // 128, K // 128), torch.float32)
        fp8.fp8_quant_weight_128x128(w.cuda(), q, s, pow2=True)
        torch.cuda.synchronize()
        check_guard(qb)
        check_guard(sbuf)
        q_ref, s_ref = quant.quant_128x128(f32(w), scale="pow2")
        assert_codes_equal(q, q_ref, what)
        assert_scales_equal(s, s_ref, what)


def test_weight_dual_and_data_gradient():
    """The dual quantiser with power-of-two scales: W and W^T codes and scales
    bit-exact against the oracle (W^T quantised on its own), and the data
    gradient dX = dY W on the scaled MFMA within the FP8 bound."""
    d = workloads.dgrad(M=200, N=384, K=768)  # dX [200, 768]: the scaled MFMA needs 256 | 768
    dy, w = d["dy"], d["w"]
    N, K = w.shape
    wpad = torch.zeros((N, K + 64), dtype=w.dtype)
    wpad[:, :K] = w  # row pitch K + 64
    say(f"pow2 dual quantiser {tuple(w.shape)} (pitch {K + 64}) and the scaled data gradient")
    bufs = [guarded(sh, dt) for sh, dt in (((N, K), torch.uint8), ((N // 128, K // 128), torch.float32),
                                           ((K, N), torch.uint8), ((K // 128, N // 128), torch.float32))]
    q, s, qt, st = (b[1] for b in bufs)
    fp8.fp8_quant_weight_128x128_dual(wpad.cuda()[:, :K], q, s, qt, st, pow2=True)
    torch.cuda.synchronize()
    for b in bufs:
        check_guard(b[0])
    rq, rs = quant.quant_128x128(f32(w), scale="pow2")
    rqt, rst = quant.quant_128x128(np.ascontiguousarray(f32(w).T), scale="pow2")
    assert_codes_equal(q, rq, "codes")
    assert_scales_equal(s, rs, "scales")
    assert_codes_equal(qt, rqt, "transposed codes")
    assert_scales_equal(st, rst, "transposed scales")
    qa, sa = fp8.fp8_quant_act_1x128(dy.cuda(), pow2=True)
    ra, rsa = quant.quant_1x128(f32(dy), scale="pow2")
    assert np.array_equal(qa.cpu().numpy(), ra) and np.array_equal(sa.cpu().numpy(), rsa)
    y = fp8.fp8_block_gemm(qa, sa, qt, st, accum="scaled", out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = gemm.block_gemm(ra, rsa, rqt, rst)
    bound = fp8_mfma_bound(ra, rsa, rqt, rst, "block")
    y = f32(y).astype(np.float64)
    say(f"  dX fp32: Frobenius {frob_rel(y, ref):.3e}, max err/bound {np.max(np.abs(y - ref) / bound):.3f}")
    assert np.all(np.isfinite(y)) and np.all(np.abs(y - ref) <= bound)


def _operands(x_cpu, w_cpu):
    qa, sa = fp8.fp8_quant_act_1x128(x_cpu.cuda(), pow2=True)
    qb, sb = fp8.fp8_quant_weight_128x128(w_cpu.cuda(), pow2=True)
    ra, rsa = quant.quant_1x128(f32(x_cpu), scale="pow2")
    rb, rsb = quant.quant_128x128(f32(w_cpu), scale="pow2")
    assert np.array_equal(qa.cpu().numpy(), ra) and np.array_equal(qb.cpu().numpy(), rb)
    assert np.array_equal(sa.cpu().numpy(), rsa) and np.array_equal(sb.cpu().numpy(), rsb)
    return (qa, sa, qb, sb), (ra, rsa, rb, rsb)


def _gemm(g, M, N, dtype):
    buf, y = guarded((M, N), dtype)
    fp8.fp8_block_gemm(*g, accum="scaled", y=y)
    torch.cuda.synchronize()
    check_guard(buf)
    return y


@pytest.mark.parametrize("M,N,K", [(300, 256, 1024), (129, 512, 384), (1, 256, 128), (64, 256, 7168),
                                   (300, 896, 1024), (129, 2688, 384)])  # N % 256 != 0: 224-wide tiles
def test_scaled_gemm_shapes(M, N, K):
    d = workloads.dense(M=M, N=N, K=K)
    g, r = _operands(d["x"], d["w"])
    ref = gemm.block_gemm(*r)
    say(f"scaled-MFMA GEMM {M}x{N}x{K}")
    y = f32(_gemm(g, M, N, torch.float32)).astype(np.float64)
    bound = fp8_mfma_bound(*r, "block")
    say(f"  fp32 out: Frobenius {frob_rel(y, ref):.3e}, max err/bound {np.max(np.abs(y - ref) / bound):.3f}")
    assert np.all(np.isfinite(y)) and np.all(np.abs(y - ref) <= bound)
    check_bf16(_gemm(g, M, N, torch.bfloat16), ref, "bf16 out")


def test_scaled_gemm_zero_tiles_and_wide_scales():
    # zero groups (scale 0), and rows scaled over a wide exponent range
    d = workloads.dense(M=130, N=256, K=512)
    x = d["x"].float().clone()
    x[5] = 0
    x[129, :256] = 0
    x[7] *= 2.0 ** 40
    x[8] *= 2.0 ** -40
    g, r = _operands(x, d["w"])
    ref = gemm.block_gemm(*r)
    y = f32(_gemm(g, 130, 256, torch.float32)).astype(np.float64)
    assert np.all(y[5] == 0)
    bound = fp8_mfma_bound(*r, "block")
    assert np.all(np.abs(y - ref) <= bound)


def test_scaled_grouped_and_gather():
    T, G, topk, N, K = 97, 8, 3, 256, 384
    logits = workloads.dense(seed=41, M=T, N=1, K=G)["x"].float().numpy()
    perm, offsets = workloads.route_topk(logits, np.zeros(G, np.float32), topk)[:2]
    x = workloads.dense(seed=42, M=T, N=128, K=K)["x"]
    w = torch.stack([workloads.moe_expert_weight(g, seed=41, N=N, K=K) for g in range(G)])
    qt, st = fp8.fp8_quant_act_1x128(x.cuda(), pow2=True)
    qb, sb = fp8.fp8_quant_weight_128x128(w.cuda().view(G * N, K), pow2=True)
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    rt, rst = quant.quant_1x128(f32(x), scale="pow2")
    assert np.array_equal(qt.cpu().numpy(), rt)
    rb = np.stack([quant.quant_128x128(f32(w[g]), scale="pow2")[0] for g in range(G)])
    rsb = np.stack([quant.quant_128x128(f32(w[g]), scale="pow2")[1] for g in range(G)])
    ref = gemm.grouped_gemm(rt[perm], rst[perm], offsets, rb, rsb)
    idx = torch.from_numpy(perm.astype(np.int32)).cuda()
    off = torch.from_numpy(offsets).cuda()
    M = int(offsets[-1])
    say(f"scaled grouped gather: {T} tokens, {G} experts top-{topk} -> {M} rows")
    y = fp8.fp8_block_grouped_gemm_gather(qt, st, idx, off, qb, sb, accum="scaled", out_dtype=torch.bfloat16)
    check_bf16(y, ref, "gather, bf16")
    yp = fp8.fp8_block_grouped_gemm(qt[idx.long()].contiguous(), st[idx.long()].contiguous(), off, qb, sb,
                                    accum="scaled", out_dtype=torch.bfloat16)
    assert torch.equal(y, yp)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_full_dense_projection_scaled():
    """4096 x 7168 x 7168 with power-of-two scales: every code and scale
    bit-exact, every bf16 output within the bf16 bound, and every fp32 output
    within the FP8-accumulation bound (its two-product form)."""
    d = workloads.dense()
    say("dense 4096x7168x7168 with power-of-two scales: quantise + scaled-MFMA GEMM")
    qa, sa = fp8.fp8_quant_act_1x128(d["x"].cuda(), pow2=True)
    qb, sb = fp8.fp8_quant_weight_128x128(d["w"].cuda(), pow2=True)
    y = fp8.fp8_block_gemm(qa, sa, qb, sb, accum="scaled")
    y32 = fp8.fp8_block_gemm(qa, sa, qb, sb, accum="scaled", out_dtype=torch.float32)
    torch.cuda.synchronize()
    ra, rsa = quant.quant_1x128(f32(d["x"]), scale="pow2")
    rb, rsb = quant.quant_128x128(f32(d["w"]), scale="pow2")
    assert_codes_equal(qa, ra, "X codes")
    assert_scales_equal(sa, rsa, "X scales")
    assert_codes_equal(qb, rb, "W codes")
    assert_scales_equal(sb, rsb, "W scales")
    say("  oracle GEMM over all rows")
    ref = gemm.block_gemm(ra, rsa, rb, rsb)
    check_bf16(y, ref, "all 4096 x 7168 outputs, bf16")
    g = f32(y32).astype(np.float64)
    bound = fp8_mfma_bound_separable(ra, rsa, rb, rsb, "block")
    err = np.abs(g - ref)
    say(f"  fp32 out, all outputs: Frobenius {frob_rel(g, ref):.3e}, max err/bound {np.max(err / bound):.3f}")
    assert np.all(np.isfinite(g)) and np.all(err <= bound)
