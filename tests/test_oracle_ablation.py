"""Per-tensor against fine-grained scaling (oracle.ablation): pins of the
per-tensor quantiser and the effect the innerforce notes' Figure 7(a)
passage describes -- outliers shrink a per-tensor scale and push small
values to E4M3's subnormal range or to zero; 1x128 / 128x128 groups confine
that to the outlier's own group."""

import numpy as np

from fp8_fine_grained_amd import workloads
from oracle import ablation, quant


def test_single_tile_tensor_is_the_tile_quantiser():
    x = workloads.dense(seed=5, M=1, N=128, K=128)["x"].float().numpy()
    qt, st = ablation.quant_per_tensor(x)
    qa, sa = quant.quant_1x128(x)
    assert np.array_equal(qt, qa) and np.float32(st) == sa[0, 0]


def test_per_tensor_invariants():
    x = workloads.quant_act(seed=4, M=32, K=512).float().numpy()
    q, s = ablation.quant_per_tensor(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[i] & 0x7F == 0x7E
    q2, s2 = ablation.quant_per_tensor(np.ldexp(x, 7).astype(np.float32))
    assert np.array_equal(q, q2) and s2 == np.float32(np.ldexp(s, 7))
    qn, sn = ablation.quant_per_tensor(-x)
    assert np.array_equal(qn, q ^ 0x80) and sn == s
    q0, s0 = ablation.quant_per_tensor(np.zeros((2, 128), np.float32))
    assert s0 == 0 and np.all(q0 == 0)


def test_outliers_hurt_per_tensor_scaling_more():
    d = workloads.dense(seed=7, M=64, N=256, K=1024)
    x, w = d["x"].float().numpy(), d["w"].float().numpy()
    r = ablation.compare(x, w)
    fine, tens = r["act_fine"], r["act_tensor"]
    # values below E4M3's normal range (or zero): far fewer with 1x128 groups
    assert fine["subnormal_or_zero"] * 5 < tens["subnormal_or_zero"]
    assert fine["flushed_to_zero"] <= tens["flushed_to_zero"]
    assert fine["rel_mean"] < tens["rel_mean"]
    assert r["gemm_fine"] < r["gemm_tensor"]
    # the fine-grained GEMM error is what E4M3 rounding of both operands gives (~2-3%)
    assert r["gemm_fine"] < 0.05
