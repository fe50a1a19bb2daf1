"""Per-tensor against fine-grained scaling (oracle.ablation): pins of the
per-tensor quantiser, of the dequantisers and of the accuracy statistics,
and the effect the innerforce notes' Figure 7(a) passage describes --
outliers shrink a per-tensor scale and push small values to E4M3's
subnormal range or to zero; 1x128 / 128x128 groups confine that to the
outlier's own group.

The statistics are pinned by tests/golden/ablation_handworked.json: a 2x128
tensor (an ordinary tile and a tile holding a 64x outlier) and a two-row
weight, with every code, dequantised value, relative error, statistic and
GEMM error worked out by hand as an exact fraction."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import ablation, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ablation_handworked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _frac(s):
    return sum(Fraction(t.strip()) for t in s.split("+"))


def _matrix(spec):
    a = np.zeros(spec["shape"], np.float32)
    for r, c, v in spec["entries"]:
        a[r, c] = np.float32(float(Fraction(v)))
    return a


def _check_entries(arr, entries, what):
    for r, c, v in entries:
        want = float(_frac(v))
        assert arr[r, c] == want, f"{what}[{r},{c}] = {arr[r, c]!r}, hand-worked {v}"


def _check_codes(q, entries):
    listed = np.zeros(q.shape, bool)
    for r, c, v in entries:
        assert q[r, c] == int(v, 16), f"code[{r},{c}] = {q[r, c]:#04x}, hand-worked {v}"
        listed[r, c] = True
    assert np.all(q[~listed] == 0), "unlisted +0.0 entries must quantise to 0x00"


def stat_mismatches(stats, expected):
    """Names of the statistics that differ from the hand-worked fractions."""
    bad = []
    for k, v in expected.items():
        want = float(_frac(v))
        got = stats[k]
        if not (got == want or (want != 0 and abs(got - want) <= 1e-12 * abs(want))):
            bad.append((k, got, v))
    return bad


def _fine_and_tensor(g, qdq=ablation.qdq_stats):
    x = _matrix(g["x"])
    qa, sa = quant.quant_1x128(x)
    qt, st = ablation.quant_per_tensor(x)
    fine = quant.dequant_1x128(qa, sa)
    tens = ablation.dequant_per_tensor(qt, st)
    return x, (qa, sa, fine, {**qdq(x, fine), "subnormal_or_zero": ablation.subnormal_fraction(qa, x)}), (
        qt, st, tens, {**qdq(x, tens), "subnormal_or_zero": ablation.subnormal_fraction(qt, x)})


def test_handworked_codes_and_dequantised_values():
    g = _golden()
    x, (qa, sa, fine, _), (qt, st, tens, _) = _fine_and_tensor(g)
    assert [float(v) for v in sa[:, 0]] == [float(_frac(s)) for s in g["fine"]["scales"]]
    assert float(st) == float(_frac(g["tensor"]["scale"]))
    _check_codes(qa, g["fine"]["codes"])
    _check_codes(qt, g["tensor"]["codes"])
    _check_entries(fine, g["fine"]["deq"], "1x128 deq")
    _check_entries(tens, g["tensor"]["deq"], "per-tensor deq")
    # the element-wise relative errors behind the statistics
    for side, deq in (("fine", fine), ("tensor", tens)):
        for r, c, v in g[side]["rel"]:
            got = abs(deq[r, c] - np.float64(x[r, c])) / abs(np.float64(x[r, c]))
            assert math.isclose(got, float(_frac(v)), rel_tol=1e-15, abs_tol=0), (side, r, c, got, v)


def test_handworked_statistics():
    g = _golden()
    _, (_, _, _, fine_stats), (_, _, _, tens_stats) = _fine_and_tensor(g)
    assert stat_mismatches(fine_stats, g["fine"]["stats"]) == []
    assert stat_mismatches(tens_stats, g["tensor"]["stats"]) == []


def test_handworked_gemm_error():
    g = _golden()
    x, w = _matrix(g["x"]), _matrix(g["w"])
    qb, sb = quant.quant_128x128(w)
    wf = quant.dequant_128x128(qb, sb)
    assert np.array_equal(wf, w.astype(np.float64)), "W is E4M3-exact with s = 1"
    qw, sw = ablation.quant_per_tensor(w)
    assert np.array_equal(ablation.dequant_per_tensor(qw, sw), w.astype(np.float64))
    _, (_, _, fine, _), (_, _, tens, _) = _fine_and_tensor(g)
    gg = g["gemm"]
    ref_norm = math.sqrt(float(_frac(gg["ref_sq_norm"])))
    want_fine = math.sqrt(float(_frac(gg["fine_err_sq_norm"]))) / ref_norm
    want_tens = math.sqrt(float(_frac(gg["tensor_err_sq_norm"]))) / ref_norm
    assert math.isclose(ablation.gemm_error(x, w, fine, wf), want_fine, rel_tol=1e-12)
    assert math.isclose(ablation.gemm_error(x, w, tens, wf), want_tens, rel_tol=1e-12)
    # compare() reports the same figures
    r = ablation.compare(x, w)
    assert math.isclose(r["gemm_fine"], want_fine, rel_tol=1e-12)
    assert math.isclose(r["gemm_tensor"], want_tens, rel_tol=1e-12)
    assert stat_mismatches(r["act_fine"], g["fine"]["stats"]) == []
    assert stat_mismatches(r["act_tensor"], g["tensor"]["stats"]) == []


@pytest.mark.parametrize("case", _golden()["dequant_cases"], ids=lambda c: c["kind"])
def test_handworked_dequant_scale_indexing(case):
    x = _matrix(case)
    if case["kind"] == "act_1x128":
        q, s = quant.quant_1x128(x)
        deq = quant.dequant_1x128(q, s)
        scales = s[0]
    else:
        q, s = quant.quant_128x128(x)
        deq = quant.dequant_128x128(q, s)
        scales = s[0]
    assert [float(v) for v in scales] == [float(_frac(v)) for v in case["scales"]]
    _check_entries(deq, case["deq"], case["kind"] + " deq")
    listed = np.zeros(x.shape, bool)
    for r, c, _ in case["deq"]:
        listed[r, c] = True
    assert np.all(deq[~listed] == 0)


@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
def test_planted_mistake_fails_the_pins():
    """The fixture catches a plausible slip in the statistics: the relative
    error taken against the dequantised value instead of the input (elements
    flushed to zero make that ratio infinite, so its percentiles warn)."""
    def wrong_qdq(x, deq):
        x = np.asarray(x, np.float64)
        deq = np.asarray(deq, np.float64)
        nz = x != 0
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.abs(deq[nz] - x[nz]) / np.abs(deq[nz])
        return {"rel_median": float(np.median(rel)), "rel_p99": float(np.percentile(rel, 99)),
                "rel_mean": float(np.mean(rel)), "flushed_to_zero": float(np.mean(deq[nz] == 0)),
                "frac_nonzero": float(np.mean(nz))}

    g = _golden()
    _, (_, _, _, fine_stats), (_, _, _, tens_stats) = _fine_and_tensor(g, qdq=wrong_qdq)
    assert stat_mismatches(fine_stats, g["fine"]["stats"]) != []
    assert stat_mismatches(tens_stats, g["tensor"]["stats"]) != []


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
