"""GPU parity of the GEMM whose output leaves quantised 1x128 (fp8_block_gemm_quant).

Against the oracle: the fused kernel quantises its own fp32 accumulators, which
differ from the fp64 product by at most the FP8-accumulation bound b
(tests.gpu_util.fp8_mfma_bound).  So, per row and 1x128 group of the output:
  * the scale is within b/448 of amax(ref)/448 (amax is 1-Lipschitz), and a
    power-of-two scale s brackets the group: amax(ref) - b <= 448 s and
    amax(ref) + b > 224 s;
  * every dequantised element is within 2^-4 |y| + 2^-10 s (the cast's QDQ
    bound) + b of the reference.
Against the library itself (an invariant, not a parity claim): the fused codes
and scales equal, bit for bit, the fp32-output GEMM followed by the 1x128
quantiser, since both run the same accumulation.
"""

import numpy as np
import pytest
import torch

import workloads
from fp8_fine_grained_amd import binding as fp8
from oracle import e4m3, gemm, quant
from tests.gpu_util import check_guard, f32, fp8_mfma_bound, fp8_mfma_bound_separable, guarded, say

pytestmark = pytest.mark.gpu


def _operands(x_cpu, w_cpu, pow2):
    qa, sa = fp8.fp8_quant_act_1x128(x_cpu.cuda(), pow2=pow2)
    qb, sb = fp8.fp8_quant_weight_128x128(w_cpu.cuda(), pow2=pow2)
    scale = "pow2" if pow2 else "amax"
    ra, rsa = quant.quant_1x128(f32(x_cpu), scale=scale)
    rb, rsb = quant.quant_128x128(f32(w_cpu), scale=scale)
    assert np.array_equal(qa.cpu().numpy(), ra) and np.array_equal(qb.cpu().numpy(), rb)
    return (qa, sa, qb, sb), (ra, rsa, rb, rsb)


def _check_against_oracle(q, s, ref, bound, pow2, what):
    q = q.cpu().numpy() if isinstance(q, torch.Tensor) else q
    s = s.cpu().numpy().astype(np.float64) if isinstance(s, torch.Tensor) else s.astype(np.float64)
    M, N = ref.shape
    G = N // 128
    refg = ref.reshape(M, G, 128)
    bg = bound.reshape(M, G, 128).max(axis=2)
    amax = np.abs(refg).max(axis=2)
    if pow2:
        m, _ = np.frexp(s[s != 0])
        assert np.all(m == 0.5), f"{what}: scale not a power of two"
        assert np.all(amax - bg <= 448 * s * (1 + 1e-12)) and np.all(amax + bg > 224 * s), f"{what}: pow2 bracket"
    else:
        err_s = np.abs(s - amax / 448)
        assert np.all(err_s <= bg / 448 + amax / 448 * 2.0 ** -22), f"{what}: scale off by {np.max(err_s):.3e}"
    deq = e4m3.decode(q).reshape(M, G, 128) * s[:, :, None]
    tol = 2.0 ** -4 * (np.abs(refg) + bound.reshape(M, G, 128)) + 2.0 ** -10 * s[:, :, None] + bound.reshape(M, G, 128)
    err = np.abs(deq - refg)
    say(f"  {what}: max err/tol {np.max(err / tol):.3f}, rel Frobenius of deq {np.linalg.norm(deq - refg) / np.linalg.norm(refg):.2e}")
    assert np.all(err <= tol), f"{what}: dequantised output outside the bound"


@pytest.mark.parametrize("M,N,K,pow2", [(300, 512, 1024, False), (129, 256, 384, False), (64, 256, 7168, False),
                                        (300, 512, 1024, True), (1, 256, 128, True)])
def test_fused_quant_against_oracle(M, N, K, pow2):
    d = workloads.dense(M=M, N=N, K=K)
    g, r = _operands(d["x"], d["w"], pow2)
    accum = "scaled" if pow2 else "fp8"
    say(f"fused GEMM + 1x128 quantisation {M}x{N}x{K} ({accum}, {'pow2' if pow2 else 'amax/448'} scales)")
    qbuf, q = guarded((M, N), torch.uint8)
    sbuf, s = guarded((M, N // 128), torch.float32)
    fp8.fp8_block_gemm_quant(*g, accum=accum, pow2=pow2, q=q, scales=s)
    torch.cuda.synchronize()
    check_guard(qbuf)
    check_guard(sbuf)
    ref = gemm.block_gemm(*r)
    _check_against_oracle(q, s, ref, fp8_mfma_bound(*r, "block"), pow2, "fused output")


@pytest.mark.parametrize("pow2", [False, True])
def test_fused_equals_gemm_then_quantiser(pow2):
    d = workloads.dense(M=517, N=768, K=896)
    g, _ = _operands(d["x"], d["w"], pow2)
    accum = "scaled" if pow2 else "fp8"
    q, s = fp8.fp8_block_gemm_quant(*g, accum=accum, pow2=pow2)
    y32 = fp8.fp8_block_gemm(*g, accum=accum, out_dtype=torch.float32)
    q2, s2 = fp8.fp8_quant_act_1x128(y32, pow2=pow2)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_full_dense_projection_fused():
    """4096 x 7168 x 7168 with the output cast to E4M3 1x128 in the GEMM: every
    input code bit-exact, and every output group's scale and every output code
    within the bounds above, with b the FP8-accumulation bound in its
    two-product form (an upper bound of the per-run form)."""
    d = workloads.dense()
    say("dense 4096x7168x7168: quantise X, W; GEMM with the output cast to E4M3 1x128")
    g = (*fp8.fp8_quant_act_1x128(d["x"].cuda()), *fp8.fp8_quant_weight_128x128(d["w"].cuda()))
    q, s = fp8.fp8_block_gemm_quant(*g)
    torch.cuda.synchronize()
    ra, rsa = quant.quant_1x128(f32(d["x"]))
    rb, rsb = quant.quant_128x128(f32(d["w"]))
    assert np.array_equal(g[0].cpu().numpy(), ra) and np.array_equal(g[2].cpu().numpy(), rb)
    say("  oracle GEMM and bound over all rows")
    ref = gemm.block_gemm(ra, rsa, rb, rsb)
    _check_against_oracle(q, s, ref, fp8_mfma_bound_separable(ra, rsa, rb, rsb, "block"), False,
                          "all 4096 x 7168 outputs")
