"""Seeded randomized sweep of the quantisers: random shapes, row pitches,
input types (fp32, bf16), transposed reads and both scale rules (amax/448 and
power of two), every code and scale compared bit for bit with the oracle."""

import numpy as np
import pytest
import torch

from fp8_fine_grained_amd import binding as fp8
from oracle import quant
from tests.gpu_util import assert_codes_equal, assert_scales_equal, f32, say

pytestmark = pytest.mark.gpu


def _draw(rng, shape, kind):
    """Values with the structure the quantisers must handle: normal rows, heavy
    tails, rows of zeros, single outliers and wide per-row magnitude spreads."""
    x = rng.standard_normal(shape).astype(np.float32)
    if kind == "heavy":
        x = (x / np.sqrt(rng.chisquare(3, shape) / 3)).astype(np.float32)
    elif kind == "spread":
        x *= np.exp2(rng.integers(-30, 30, (shape[0], 1))).astype(np.float32)
    r = rng.integers(0, shape[0])
    x[r] = 0
    x[rng.integers(0, shape[0]), rng.integers(0, shape[1])] *= 1000
    return x


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(dict(i=i, what=["rows", "cols", "weight", "dual", "act_weight"][i % 5],
                        M=int(rng.integers(1, 600)), K=128 * int(rng.integers(1, 12)),
                        N=128 * int(rng.integers(1, 6)), pad=int(rng.integers(0, 4)) * 64,
                        dtype=["fp32", "bf16"][int(rng.integers(0, 2))], pow2=bool(rng.random() < 0.4),
                        kind=["normal", "heavy", "spread"][int(rng.integers(0, 3))]))
    return out


@pytest.mark.parametrize("c", _cases(30, 77), ids=lambda c: "{i}_{what}_{dtype}_{kind}{p}".format(
    p="_pow2" if c["pow2"] and c["what"] != "dual" else "", **c))
def test_quantiser_sweep(c):
    rng = np.random.default_rng(1000 + c["i"])
    tdt = torch.float32 if c["dtype"] == "fp32" else torch.bfloat16
    scale = "pow2" if c["pow2"] else "amax"
    M, K, N, pad = c["M"], c["K"], c["N"], c["pad"]
    say(f"case {c}")
    if c["what"] in ("rows", "act_weight"):
        base = torch.from_numpy(_draw(rng, (M, K + pad), c["kind"])).to(tdt)
        x = base[:, :K]  # row pitch K + pad elements
        if c["what"] == "rows":
            q, s = fp8.fp8_quant_act_1x128(base.cuda()[:, :K], pow2=c["pow2"])
        else:
            wb = torch.from_numpy(_draw(rng, (N, K + pad), c["kind"])).to(tdt)
            q, s, qw, sw = fp8.fp8_quant_act_weight(base.cuda()[:, :K], wb.cuda()[:, :K], pow2=c["pow2"])
            rw, rsw = quant.quant_128x128(f32(wb[:, :K]), scale=scale)
            assert_codes_equal(qw, rw, "weight codes")
            assert_scales_equal(sw, rsw, "weight scales")
        r, rs = quant.quant_1x128(f32(x), scale=scale)
    elif c["what"] == "cols":
        M = 8 * ((M + 7) // 8)  # the transposed read takes whole 16-byte runs of tokens
        base = torch.from_numpy(_draw(rng, (K, M + pad), c["kind"])).to(tdt)
        xt = base.cuda()[:, :M].t()  # logical [M, K], tiles along the strided axis
        q, s = fp8.fp8_quant_act_1x128(xt, pow2=c["pow2"])
        r, rs = quant.quant_1x128(np.ascontiguousarray(f32(base[:, :M]).T), scale=scale)
    else:
        Nw = 128 * max(1, M // 128)
        base = torch.from_numpy(_draw(rng, (Nw, K + pad), c["kind"])).to(tdt)
        if c["what"] == "weight":
            q, s = fp8.fp8_quant_weight_128x128(base.cuda()[:, :K], pow2=c["pow2"])
        else:
            scale = "amax"  # the dual quantiser has the amax/448 rule only
            q, s, qt, st = fp8.fp8_quant_weight_128x128_dual(base.cuda()[:, :K])
            rt, rst = quant.quant_128x128(np.ascontiguousarray(f32(base[:, :K]).T))
            assert_codes_equal(qt, rt, "transposed codes")
            assert_scales_equal(st, rst, "transposed scales")
        r, rs = quant.quant_128x128(f32(base[:, :K]), scale=scale)
    torch.cuda.synchronize()
    assert_codes_equal(q, r, "codes")
    assert_scales_equal(s, rs, "scales")
