"""GPU parity of the per-tensor quantiser (one scale for the whole tensor, the
practice the 1x128 / 128x128 grouping replaces) against the oracle's
per-tensor quantiser: codes and the scale bit for bit, the scale in every
entry of the requested layout, and the block GEMM on per-tensor operands."""

import numpy as np
import pytest
import torch

import workloads
from fp8_fine_grained_amd import binding as fp8
from oracle import ablation, gemm
from tests.gpu_util import assert_codes_equal, check_bf16, f32, say

pytestmark = pytest.mark.gpu


def _check(x_cpu, layout, what):
    say(f"per-tensor {what} {tuple(x_cpu.shape)} {layout}")
    q, s = fp8.fp8_quant_per_tensor(x_cpu.cuda(), layout=layout)
    torch.cuda.synchronize()
    q_ref, s_ref = ablation.quant_per_tensor(f32(x_cpu))
    assert_codes_equal(q, q_ref, what)
    M, K = x_cpu.shape
    assert s.shape == ((M if layout == "act" else M // 128), K // 128)
    got = s.cpu().numpy().view(np.uint32)
    assert np.all(got == np.float32(s_ref).view(np.uint32)), f"{what}: scales differ from {s_ref}"
    return q, s, q_ref, s_ref


def test_activation_layout():
    d = workloads.dense(M=300, N=128, K=1024)  # 0.1% of entries x100
    _check(d["x"], "act", "dense-like bf16")
    _check(workloads.tiny()["x"], "act", "tiny fp32 (1% x50)")


def test_padded_row_pitch():
    # x is the first 512 columns of a [256, 640] tensor: row pitch 640 elements
    wide = workloads.dense(M=256, N=128, K=640)["x"]
    x = wide.cuda()[:, :512]
    say(f"per-tensor padded pitch {tuple(x.shape)} ld {x.stride(0)}")
    q, s = fp8.fp8_quant_per_tensor(x)
    torch.cuda.synchronize()
    q_ref, s_ref = ablation.quant_per_tensor(f32(wide[:, :512].contiguous()))
    assert_codes_equal(q, q_ref, "padded pitch")
    assert np.all(s.cpu().numpy().view(np.uint32) == np.float32(s_ref).view(np.uint32))


def test_weight_layout():
    _check(workloads.dense(M=1, N=384, K=1024)["w"], "weight", "weight bf16")
    _check(workloads.tiny()["w"], "weight", "tiny weight fp32")


def test_zero_and_signed_zero():
    x = torch.zeros((128, 256), dtype=torch.float32)
    x[3, 5] = -0.0
    q, s = fp8.fp8_quant_per_tensor(x.cuda())
    torch.cuda.synchronize()
    assert torch.all(s == 0)
    qc = q.cpu()
    assert qc[3, 5] == 0x80 and int((qc != 0).sum()) == 1


def test_full_dense_activation():
    # [4096, 7168]: 229376 tiles, 2048 amax blocks striding over them
    _check(workloads.dense()["x"], "act", "dense projection X")


def test_gemm_on_per_tensor_operands():
    d = workloads.dense(M=300, N=512, K=1024)
    qa, sa, ra, rsa = _check(d["x"], "act", "X")
    qb, sb, rb, rsb = _check(d["w"], "weight", "W")
    y = fp8.fp8_block_gemm(qa, sa, qb, sb, accum="fp8", out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    M, K = d["x"].shape
    N = d["w"].shape[0]
    ref = gemm.block_gemm(ra, np.full((M, K // 128), rsa, np.float32), rb,
                          np.full((N // 128, K // 128), rsb, np.float32))
    check_bf16(y, ref, "GEMM on per-tensor operands")
