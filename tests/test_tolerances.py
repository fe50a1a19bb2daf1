"""CPU checks of the GPU tests' tolerance helpers (tests/gpu_util.py)."""

import numpy as np
import pytest

from tests.gpu_util import fp8_mfma_bound, fp8_mfma_bound_loops


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
