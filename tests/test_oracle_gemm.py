"""Pins for oracle.gemm: exact rational brute force on tiny shapes, exact
integer matmul when every scale is one, the closed form for K = 128,
linearity in each scale block, and grouped == per-segment dense."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm
from tests.exact import e4m3_values_torch

DEC = e4m3_values_torch()


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x41
    return c


def _scales(rng, shape):
    # fp32 scales spanning several binades, with arbitrary mantissas
    return (rng.uniform(0.5, 2.0, size=shape) * 2.0 ** rng.integers(-12, 4, size=shape)).astype(np.float32)


def _brute(qa, sa, qb, sb, mode):
    M, K = qa.shape
    N = qb.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                a = Fraction(DEC[qa[m, k]]) * Fraction(float(sa[m, k // 128]))
                sbv = sb[n // 128, k // 128] if mode == "block" else sb[n, k // 128]
                b = Fraction(DEC[qb[n, k]]) * Fraction(float(sbv))
                acc += a * b
            out[m, n] = float(acc)
    return out


@pytest.mark.parametrize("mode,M,N,K", [("block", 3, 136, 256), ("row", 4, 5, 384), ("block", 2, 256, 128)])
def test_brute_force_exact_rationals(mode, M, N, K):
    rng = np.random.default_rng(31 + M)
    qa, qb = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = _scales(rng, (M, K // 128))
    sb = _scales(rng, ((N + 127) // 128 if mode == "block" else N, K // 128))
    got = gemm.block_gemm(qa, sa, qb, sb, mode)
    want = _brute(qa, sa, qb, sb, mode)
    scale = np.abs(want).max()
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13 * scale)


def test_unit_scales_reduce_to_exact_integer_matmul():
    rng = np.random.default_rng(40)
    M, N, K = 48, 256, 512
    qa, qb = _codes(rng, (M, K)), _codes(rng, (N, K))
    ia = np.array([int(DEC[c] * 512) for c in range(256) if (c & 0x7F) != 0x7F] + [0, 0])
    to_int = np.zeros(256, np.int64)
    to_int[[c for c in range(256) if (c & 0x7F) != 0x7F]] = ia[:-2]
    ya = to_int[qa]
    yb = to_int[qb]
    exact = ya @ yb.T  # int64, exact: each |term| < 2^36, sums < 2^46
    got = gemm.block_gemm(qa, np.ones((M, K // 128), np.float32), qb, np.ones((2, K // 128), np.float32))
    assert np.array_equal(got * 2.0 ** 18, exact.astype(np.float64))


def test_single_block_closed_form():
    rng = np.random.default_rng(41)
    M, N, K = 16, 128, 128
    qa, qb = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa, sb = _scales(rng, (M, 1)), _scales(rng, (1, 1))
    da = np.array([[DEC[c] for c in row] for row in qa])
    db = np.array([[DEC[c] for c in row] for row in qb])
    P = da @ db.T  # exact: integer multiples of 2^-18 below 2^53
    want = P * (sa.astype(np.float64) * np.float64(sb[0, 0]))
    got = gemm.block_gemm(qa, sa, qb, sb)
    bound = (np.abs(da) @ np.abs(db).T) * (sa.astype(np.float64) * np.float64(sb[0, 0])) * K * 2.0 ** -52
    assert np.all(np.abs(got - want) <= bound)


def test_linear_in_each_scale_block():
    rng = np.random.default_rng(42)
    M, N, K = 8, 256, 384
    qa, qb = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa, sb = _scales(rng, (M, 3)), _scales(rng, (2, 3))
    y0 = gemm.block_gemm(qa, sa, qb, sb)
    sb2 = sb.copy()
    sb2[1, 2] *= 2  # doubles the contribution of k-block 2 to outputs n in [128, 256)
    y1 = gemm.block_gemm(qa, sa, qb, sb2)
    only = np.zeros_like(sb)
    only[1, 2] = sb[1, 2]
    contrib = gemm.block_gemm(qa, sa, qb, only)
    assert np.allclose(y1 - y0, contrib, rtol=1e-12, atol=1e-12 * np.abs(y0).max())
    assert np.all(contrib[:, :128] == 0)


def _grouped_case(rng, G, sizes, N=256, K=256):
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(sizes)
    M = int(offsets[-1])
    qa = _codes(rng, (M, K))
    sa = _scales(rng, (M, K // 128))
    qb = _codes(rng, (G, N, K))
    sb = _scales(rng, (G, N // 128, K // 128))
    return qa, sa, offsets, qb, sb


def test_grouped_equals_per_segment_dense():
    rng = np.random.default_rng(43)
    sizes = [5, 0, 1, 17, 0, 9]
    qa, sa, off, qb, sb = _grouped_case(rng, len(sizes), sizes)
    y = gemm.grouped_gemm(qa, sa, off, qb, sb)
    for g in range(len(sizes)):
        r0, r1 = off[g], off[g + 1]
        if r1 > r0:
            ref = gemm.block_gemm(qa[r0:r1], sa[r0:r1], qb[g], sb[g])
            assert np.allclose(y[r0:r1], ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    # a brute-force spot check of one row of each non-empty segment
    for g in range(len(sizes)):
        if off[g + 1] > off[g]:
            m = int(off[g])
            want = _brute(qa[m:m + 1], sa[m:m + 1], qb[g][:3], sb[g][:1], "block")
            assert np.allclose(y[m, :3], want[0], rtol=1e-13, atol=1e-13 * np.abs(want).max())


def test_grouped_single_group_is_dense_and_rows_subset():
    rng = np.random.default_rng(44)
    qa, sa, off, qb, sb = _grouped_case(rng, 1, [23])
    y = gemm.grouped_gemm(qa, sa, off, qb, sb)
    ref = gemm.block_gemm(qa, sa, qb[0], sb[0])
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    qa, sa, off, qb, sb = _grouped_case(rng, 4, [3, 0, 8, 2])
    full = gemm.grouped_gemm(qa, sa, off, qb, sb)
    rows = np.array([12, 0, 5, 3])
    sub = gemm.grouped_gemm(qa, sa, off, qb, sb, rows=rows)
    assert np.allclose(sub, full[rows], rtol=1e-13, atol=1e-13 * np.abs(full).max())


def test_grouped_rejects_bad_offsets():
    rng = np.random.default_rng(45)
    qa, sa, off, qb, sb = _grouped_case(rng, 3, [2, 2, 2])
    with pytest.raises(ValueError):
        gemm.grouped_gemm(qa, sa, np.array([0, 4, 2, 6]), qb, sb)
