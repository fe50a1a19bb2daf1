"""CPU checks of the GPU tests' tolerance helpers (tests/gpu_util.py)."""

import numpy as np
import pytest

from tests.gpu_util import fp8_mfma_bound, fp8_mfma_bound_loops, fp8_mfma_bound_separable


@pytest.mark.parametrize("mode", ["block", "row"])
def test_fast_fp8_accumulation_bound_equals_the_loop_form(mode):
    rng = np.random.default_rng(11)
    M, N, K = 37, 256, 384
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    # no NaN codes; plenty of zeros (whole zero runs included) and subnormals
    for q in (qa, qb):
        q[(q & 0x7F) == 0x7F] = 0x7E
        q[rng.random(q.shape) < 0.2] = 0
        q[:, 8:16] = 0
        q[rng.random(q.shape) < 0.1] &= 0x87
    sa = rng.uniform(0.5, 2.0, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.5, 2.0, ((N // 128) if mode == "block" else N, K // 128)).astype(np.float32)
    fast = fp8_mfma_bound(qa, sa, qb, sb, mode, row_chunk=16)
    ref = fp8_mfma_bound_loops(qa, sa, qb, sb, mode)
    assert np.allclose(fast, ref, rtol=1e-12, atol=0)
    assert np.all(fast[:, :] > 0)


@pytest.mark.parametrize("mode", ["block", "row"])
@pytest.mark.parametrize("kind", ["uniform codes", "normal data"])
def test_separable_bound_is_an_upper_bound(mode, kind):
    """The two-product form used over whole full-size outputs never falls below
    the per-run form, element by element (zero runs, subnormals and one-sided
    zero runs included), and stays within a small factor of it on data shaped
    like the workloads'."""
    rng = np.random.default_rng(12)
    M, N, K = 40, 256, 512
    if kind == "uniform codes":
        qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
        qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
        for q in (qa, qb):
            q[(q & 0x7F) == 0x7F] = 0x7E
            q[rng.random(q.shape) < 0.2] = 0
            q[rng.random(q.shape) < 0.1] &= 0x87
        qa[:, 8:16] = 0       # runs with no nonzero A code
        qb[:, 24:32] = 0      # and with none on the B side
        qa[:, 40:44] = 0      # one-sided zeros inside a run
        qb[:, 44:48] = 0
    else:
        from oracle import quant

        xa = rng.standard_normal((M, K)).astype(np.float32)
        xb = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        qa, _ = quant.quant_1x128(xa)
        qb, _ = quant.quant_1x128(xb) if mode == "row" else quant.quant_128x128(xb)
    sa = rng.uniform(0.5, 2.0, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.5, 2.0, ((N // 128) if mode == "block" else N, K // 128)).astype(np.float32)
    tight = fp8_mfma_bound(qa, sa, qb, sb, mode, row_chunk=16)
    sep = fp8_mfma_bound_separable(qa, sa, qb, sb, mode)
    assert np.all(sep >= tight * (1 - 1e-12))
    ratio = float(np.median(sep / tight))
    assert ratio < (16.0 if kind == "uniform codes" else 4.0), ratio  # 1.55 measured on the normal data
