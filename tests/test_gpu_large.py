"""Operands past 4 GiB: the quantisers and the GEMMs address A with 64-bit row
offsets.  An activation of 524325 x 8192 bf16 (4.30e9 elements, so its E4M3
codes end past byte 2^32) is quantised 1x128 and multiplied by 256-row
weights: dense (256 x 256 tiles, FP8 accumulation, bf16 out; a ragged last
m-tile of 37 rows) and grouped over three ragged experts (exact accumulation,
fp32 out; a segment boundary sits two rows past the 2^32-byte boundary).  Rows on both
sides of that boundary, at tile edges and at the ragged end are checked
against the oracle: codes and scales bit for bit, outputs within the
bf16 bound and the fp32 1e-5 Frobenius bound."""

import numpy as np
import pytest
import torch

import workloads
from fp8_fine_grained_amd import binding as fp8
from oracle import gemm, quant
from tests.gpu_util import check_bf16, check_f32, say

pytestmark = pytest.mark.gpu

M, K, N = 524325, 8192, 256  # M * K = 4,295,270,400 > 2^32
EDGE = (1 << 32) // K  # 524288: the first row whose codes start at byte 2^32
# M - EDGE = 37: the last dense m-tile (256 rows) starts at EDGE and holds 37
OFFSETS = [0, 200003, EDGE + 2, M]  # three experts; the second ends 2 rows past byte 2^32
ROWS = [0, 1, 255, 256, 262143, EDGE - 65, EDGE - 1, EDGE, EDGE + 1, EDGE + 2, EDGE + 18, M - 1]
assert all(0 <= r < M for r in ROWS) and len(set(ROWS)) == len(ROWS)


def take_rows(t):
    """The sampled rows, each copied to the host as a contiguous slice (no
    device indexing kernel: torch's gather faults on a tensor this large)."""
    return np.concatenate([t[r:r + 1].cpu().numpy() for r in ROWS])


@pytest.fixture(scope="module")
def big():
    say(f"operands past 4 GiB: X bf16 [{M},{K}] ({M * K} elements), W bf16 [{N},{K}]")
    gen = torch.Generator(device="cuda").manual_seed(17)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, M, 1 << 16):
        r1 = min(M, r0 + (1 << 16))
        x[r0:r1] = torch.randn((r1 - r0, K), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    qa, sa = fp8.fp8_quant_act_1x128(x)
    torch.cuda.synchronize()
    x_rows = take_rows(x.view(torch.int16)).view(np.uint16)
    x_rows = (x_rows.astype(np.uint32) << 16).view(np.float32)  # bf16 -> fp32, exact
    del x
    return qa, sa, x_rows


def test_quantiser_rows_past_4gib(big):
    qa, sa, x_rows = big
    r, rs = quant.quant_1x128(x_rows)
    q_rows, s_rows = take_rows(qa), take_rows(sa)
    bad = np.argwhere(q_rows != r)
    assert bad.size == 0, f"{bad.shape[0]} code mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(s_rows.view(np.uint32), rs.view(np.uint32)), "scales of the sampled rows differ"


def test_dense_gemm_rows_past_4gib(big):
    qa, sa, _ = big
    w = workloads.dense(seed=18, M=16, N=N, K=K)["w"]
    qb, sb = fp8.fp8_quant_weight_128x128(w.cuda())
    y = fp8.fp8_block_gemm(qa, sa, qb, sb, accum="fp8", out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = gemm.block_gemm(take_rows(qa), take_rows(sa), qb.cpu().numpy(), sb.cpu().numpy())
    y_rows = (take_rows(y.view(torch.int16)).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    check_bf16(y_rows.astype(np.float64), ref, "dense GEMM, sampled rows")


def test_grouped_gemm_rows_past_4gib(big):
    qa, sa, _ = big
    G = len(OFFSETS) - 1
    w = torch.stack([workloads.moe_expert_weight(g, seed=19, N=N, K=K) for g in range(G)])
    qb, sb = fp8.fp8_quant_weight_128x128(w.cuda().view(G * N, K))
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    off = torch.tensor(OFFSETS, dtype=torch.int32, device="cuda")
    y = fp8.fp8_block_grouped_gemm(qa, sa, off, qb, sb, accum="exact", out_dtype=torch.float32)
    torch.cuda.synchronize()
    qa_r, sa_r = take_rows(qa), take_rows(sa)
    qb_h, sb_h = qb.cpu().numpy(), sb.cpu().numpy()
    ref = np.empty((len(ROWS), N))
    for i, m in enumerate(ROWS):
        g = int(np.searchsorted(OFFSETS, m, side="right")) - 1
        ref[i] = gemm.block_gemm(qa_r[i:i + 1], sa_r[i:i + 1], qb_h[g], sb_h[g])[0]
    check_f32(take_rows(y).astype(np.float64), ref, "grouped GEMM (exact), sampled rows")
