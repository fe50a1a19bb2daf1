"""Reference for the block-scaled FP8 GEMM, dense and grouped.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

The GEMM multiplies the dequantised operands.  The pages describe how the
product is carried out on the device -- FP8 multiply-accumulate whose
partials are promoted to FP32 every 128 elements of K, with the group scales
applied at that promotion (DeepSeek-V3 FP8 training notes, accumulation
passage; yunhecapital.com report section 2.2.3; tonho.wtf "DeepSeek-V3",
"como funciona").  That schedule only changes rounding: the quantity it
approximates is the plain product of the dequantised matrices, which is what
this module computes, in fp64:

    Y[m, n] = sum_k  dec(qa[m,k]) * sa[m, k//128]  *  dec(qb[n,k]) * sb(n, k//128)

with ``sb(n, kb) = sb[n//128, kb]`` for 128x128-quantised weights ("block"
mode) and ``sb(n, kb) = sb[n, kb]`` for a 1x128-quantised second operand
("row" mode, the weight-gradient GEMM whose operands are both gradient-style
1x128 tiles, tonho.wtf "DeepSeek-V3", "o que isso custou").  Y = A * B^T with
both operands stored K-contiguous, as a linear layer's Y = X W^T.

Every dequantised value is an FP8 grid value times an fp32 scale, exact in
fp64; the fp64 matmul then rounds at ~1e-16 relative per term, far below the
fp32-accumulation error of the method.

Grouped GEMM (mixture-of-experts): rows ``offsets[g] .. offsets[g+1]-1`` of
A are the tokens routed to expert g and are multiplied by expert g's weight
``qb[g]``.  No token is dropped, so segments have arbitrary lengths,
including zero (tonho.wtf "DeepSeek-V3", "como funciona"; the MoE layer with
256 routed experts and top-8 routing, yunhecapital.com report section 2.2.2).

Parity: pinned by tests/test_oracle_gemm.py (brute force in exact rational
arithmetic on tiny shapes, exact integer matmul when all scales are one,
linearity in each scale block, grouped == per-segment dense).
"""

import numpy as np

from .e4m3 import decode
from .quant import GROUP


def _deq_a(qa, sa, rows=None):
    qa = np.asarray(qa)
    sa = np.asarray(sa, np.float64)
    if rows is not None:
        qa, sa = qa[rows], sa[rows]
    K = qa.shape[1]
    return decode(qa) * np.repeat(sa, GROUP, axis=1)[:, :K]


def _deq_b(qb, sb, mode):
    qb = np.asarray(qb)
    sb = np.asarray(sb, np.float64)
    N, K = qb.shape
    if mode == "block":
        se = np.repeat(np.repeat(sb, GROUP, axis=0), GROUP, axis=1)[:N, :K]
    elif mode == "row":
        se = np.repeat(sb, GROUP, axis=1)[:, :K]
    else:
        raise ValueError("b scale mode must be 'block' or 'row'")
    return decode(qb) * se


def block_gemm(qa, sa, qb, sb, mode="block", rows=None):
    """fp64 Y = deq(A) deq(B)^T; ``rows`` (optional index array) selects rows of Y."""
    a = _deq_a(qa, sa, rows)
    b = _deq_b(qb, sb, mode)
    return a @ b.T


def grouped_gemm(qa, sa, offsets, qb, sb, rows=None):
    """fp64 grouped GEMM over expert row segments.

    ``qb`` [G, N, K] and ``sb`` [G, N/128, K/128] (block mode per expert);
    ``offsets`` [G+1] non-decreasing with offsets[0] == 0.  With ``rows``
    given, only those rows of Y are computed (returned in the given order).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    G = offsets.size - 1
    if offsets[0] != 0 or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must start at 0 and be non-decreasing")
    M = int(offsets[-1])
    N = np.asarray(qb).shape[1]
    if rows is None:
        rows = np.arange(M)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, N), dtype=np.float64)
    expert = np.searchsorted(offsets, rows, side="right") - 1
    for g in np.unique(expert):
        sel = np.nonzero(expert == g)[0]
        out[sel] = block_gemm(qa, sa, qb[g], sb[g], "block", rows=rows[sel])
    return out
