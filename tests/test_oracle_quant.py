"""Pins for oracle.quant: hand-worked tiles, invariants the method fixes,
metamorphic relations, and each fp32 step against exact rational arithmetic."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import e4m3, quant
from tests.exact import e4m3_values_torch, round_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_tiles_handworked.json")


def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["name"])
def test_handworked_tiles(case):
    x = np.zeros(case["shape"], dtype=np.float32)
    codes = np.zeros(case["shape"], dtype=np.uint8)
    for idx, v in case["entries"]:
        x[tuple(idx) if isinstance(idx, list) else (0, idx)] = np.float32(v)
    for idx, c in case["expected_codes"]:
        codes[tuple(idx) if isinstance(idx, list) else (0, idx)] = int(c, 16)
    scale = "pow2" if case["kind"].endswith("_pow2") else "amax"
    if case["kind"].startswith("act_1x128"):
        q, s = quant.quant_1x128(x, scale=scale)
    else:
        q, s = quant.quant_128x128(x, scale=scale)
    want_s = [int(b, 16) for b in case["expected_scale_bits"]]
    assert s.reshape(-1).view(np.uint32).tolist() == want_s
    bad = np.argwhere(q != codes)
    assert bad.size == 0, [(tuple(i), hex(q[tuple(i)]), hex(codes[tuple(i)])) for i in bad[:8]]


def _inputs():
    rng = np.random.default_rng(21)
    t = workloads.quant_act(seed=3, M=64, K=384).float().numpy()
    n = workloads.dense(seed=2, M=64, N=256, K=384)["x"].float().numpy()
    tiny = workloads.tiny()["x"].numpy()
    u = rng.uniform(-3, 3, size=(64, 384)).astype(np.float32)
    return {"student_t": t, "normal_outliers": n, "tiny": tiny, "uniform": u}


INPUTS = _inputs()
DEC = np.array(e4m3_values_torch())  # independent decoder for the checks below


def _qdq_check(x, q, s_full):
    """Quantise-dequantise error: <= 2^-4 |x| in the normal range, <= 2^-10 s below it."""
    deq = DEC[q] * s_full
    err = np.abs(deq - x.astype(np.float64))
    normal = np.abs(x) >= (2.0 ** -6) * s_full
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * s_full[~normal] * (1 + 2.0 ** -20))


@pytest.mark.parametrize("name", list(INPUTS))
def test_act_invariants(name):
    x = INPUTS[name]
    q, s = quant.quant_1x128(x)
    M, K = x.shape
    assert q.dtype == np.uint8 and s.dtype == np.float32 and s.shape == (M, K // 128)
    assert not np.any((q & 0x7F) == 0x7F), "NaN code produced"
    xt = x.reshape(M, K // 128, 128)
    qt = q.reshape(M, K // 128, 128)
    amax = np.abs(xt).max(axis=2)
    # the group maximum always lands on the largest finite code
    at_max = np.abs(xt) == amax[..., None]
    assert np.all((qt[at_max] & 0x7F) == 0x7E)
    # codes other than at the maximum never exceed it
    assert np.all((qt & 0x7F) <= 0x7E)
    # scale is amax/448 to within fp32 rounding
    assert np.allclose(s, amax / 448.0, rtol=2.0 ** -23, atol=0)
    _qdq_check(x, q, np.repeat(s.astype(np.float64), 128, axis=1))


@pytest.mark.parametrize("name", list(INPUTS))
def test_weight_invariants(name):
    x = INPUTS[name][:64, :256]
    x = np.concatenate([x, x[::-1] * np.float32(0.5)], axis=0)  # [128, 256]
    q, s = quant.quant_128x128(x)
    assert s.shape == (1, 2)
    for j in range(2):
        blk = x[:, 128 * j: 128 * (j + 1)]
        qb = q[:, 128 * j: 128 * (j + 1)]
        amax = np.abs(blk).max()
        assert np.all((qb[np.abs(blk) == amax] & 0x7F) == 0x7E)
    se = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    _qdq_check(x, q, se)


@pytest.mark.parametrize("j", [-20, -3, -1, 1, 5, 30])
def test_power_of_two_equivariance(j):
    x = INPUTS["normal_outliers"]
    q0, s0 = quant.quant_1x128(x)
    q1, s1 = quant.quant_1x128(x * np.float32(2.0 ** j))
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, s0 * np.float32(2.0 ** j))
    w = x[:, :256].reshape(128, 128)
    a0, t0 = quant.quant_128x128(w)
    a1, t1 = quant.quant_128x128(w * np.float32(2.0 ** j))
    assert np.array_equal(a0, a1) and np.array_equal(t1, t0 * np.float32(2.0 ** j))


def test_sign_symmetry():
    x = INPUTS["student_t"]
    q0, s0 = quant.quant_1x128(x)
    q1, s1 = quant.quant_1x128(-x)
    assert np.array_equal(q1, q0 ^ 0x80) and np.array_equal(s0, s1)


def test_identity_on_e4m3_exact_tiles():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(32, 256)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    codes[:, 0] = 0x7E
    codes[:, 128] = 0xFE
    x = DEC[codes].astype(np.float32)
    q, s = quant.quant_1x128(x)
    assert np.all(s == 1.0)
    assert np.array_equal(q, codes)


def test_group_locality():
    x = INPUTS["uniform"].copy()
    q0, s0 = quant.quant_1x128(x)
    x[7, 200] = 1000.0  # row 7, group 1
    q1, s1 = quant.quant_1x128(x)
    ds = np.argwhere(s0 != s1)
    assert ds.tolist() == [[7, 1]]
    dq = np.argwhere(q0 != q1)
    assert np.all(dq[:, 0] == 7) and np.all((dq[:, 1] >= 128) & (dq[:, 1] < 256))
    w = INPUTS["uniform"][:, :256].reshape(128, 128).copy()
    w = np.concatenate([w, w], axis=1)  # [128, 256]: blocks (0,0), (0,1)
    a0, t0 = quant.quant_128x128(w)
    w[3, 250] = -1000.0
    a1, t1 = quant.quant_128x128(w)
    assert t0[0, 0] == t1[0, 0] and t0[0, 1] != t1[0, 1]
    assert np.array_equal(a0[:, :128], a1[:, :128])


def test_ragged_groups_cover_the_columns_present():
    x = INPUTS["student_t"][:, :300]
    q, s = quant.quant_1x128(x)
    assert s.shape == (64, 3)
    q2, s2 = quant.quant_1x128(np.ascontiguousarray(x[:, 256:]))
    assert np.array_equal(q[:, 256:], q2) and np.array_equal(s[:, 2:], s2)


def test_along_rows_is_the_transpose_case():
    x = INPUTS["normal_outliers"][:, :256]
    q, s = quant.quant_1x128_along_rows(np.ascontiguousarray(x.T))
    q2, s2 = quant.quant_1x128(x)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_weight_blocks_of_the_transpose():
    """A 128x128 block of W^T is a block of W transposed, with the same amax, so
    the block quantisation commutes with transposition (the data-gradient
    operand): codes transpose, the scale grid transposes."""
    x = workloads.dense(M=256, N=128, K=384)["x"].float().numpy()  # N(0,1) with x100 outliers
    q, s = quant.quant_128x128(x)
    assert np.any(q != q[:, ::-1])  # not trivially symmetric
    qt, st = quant.quant_128x128(np.ascontiguousarray(x.T))
    assert qt.shape == (384, 256) and st.shape == (3, 2)
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


def _near_midpoint_rows():
    """Rows whose elements sit within a few fp32 ulps of s * (E4M3 midpoint).

    Each row's first element fixes amax (a value whose scale 1/s is not a
    power of two), the rest are placed where rounding x*inv and x/s can
    disagree about which side of a midpoint y falls on."""
    rows = []
    grid = e4m3.DECODE_TABLE[:0x7F]
    mids = ((grid[:-1] + grid[1:]) / 2)[8::4]  # normal-range midpoints
    for amax in (1.0, 3.0, 0.7, 5.0e-3):
        s = np.float32(amax) / np.float32(448)
        xs = []
        for mid in mids:
            base = np.float32(mid * float(s))
            v = base
            for _ in range(2):
                v = np.nextafter(v, np.float32(-1))
            for _ in range(5):
                xs.append(v)
                v = np.nextafter(v, np.float32(1))
        xs = [x for x in xs if abs(x) < amax][:127]
        row = np.zeros(384, np.float32)
        row[0] = amax
        row[1:1 + len(xs)] = xs
        rows.append(row)
    return np.stack(rows)


def test_fp32_steps_against_exact_arithmetic():
    """s, inv and y = x*inv each rounded once in binary32, checked with rationals.

    Also confirms the rule is x*(1/s), not x/s: the set contains elements where
    the two round to different codes, and the oracle follows x*(1/s)."""
    x = np.concatenate([INPUTS["student_t"][:8], INPUTS["uniform"][:8], _near_midpoint_rows()])
    q, s = quant.quant_1x128(x)
    grid_mid = [Fraction(v) for v in e4m3_values_torch()[:0x7F]]

    def code_of(y):
        a = min(abs(y), Fraction(448))
        best = min(range(0x7F), key=lambda c: (abs(a - grid_mid[c]), c % 2))
        return best | (0x80 if y < 0 else 0)

    differs = 0
    for m in range(x.shape[0]):
        for g in range(x.shape[1] // 128):
            tile = [Fraction(float(v)) for v in x[m, 128 * g: 128 * (g + 1)]]
            amax = max(abs(v) for v in tile)
            s_ex = round_f32(amax / 448)
            assert Fraction(float(s[m, g])) == s_ex
            inv = round_f32(1 / s_ex) if s_ex else Fraction(0)
            for i in range(0, 128, 3 if m < 16 else 1):
                c_mul = code_of(round_f32(tile[i] * inv))
                c_div = code_of(round_f32(tile[i] / s_ex)) if s_ex else c_mul
                assert q[m, 128 * g + i] == c_mul
                differs += c_mul != c_div
    assert differs > 0, "test set should contain elements where x*inv and x/s differ"


def test_out_of_contract_inputs_raise():
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = np.float32(1e-38)
    with pytest.raises(ValueError):
        quant.quant_1x128(x)
    x[0, 0] = np.inf
    with pytest.raises(ValueError):
        quant.quant_1x128(x)


# ---------------------------------------------------------------- power-of-two scales


def _exponent(s):
    """e with s == 2^e exactly (asserts s is a power of two)."""
    m, e = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5), "scale is not a power of two"
    return e - 1


@pytest.mark.parametrize("name", list(INPUTS))
def test_pow2_act_invariants(name):
    x = INPUTS[name]
    q, s = quant.quant_1x128(x, scale="pow2")
    amax = np.abs(x.astype(np.float64)).reshape(x.shape[0], -1, 128).max(axis=2)
    e = _exponent(s)
    # amax / s lies in (224, 448]: exact comparisons (scaling by 2^e is exact)
    assert np.all(np.ldexp(amax, -e) <= 448.0) and np.all(np.ldexp(amax, -e) > 224.0)
    # the group's largest code sits in [0x76 (224), 0x7E (448)]; no NaN code
    top = (q & 0x7F).reshape(x.shape[0], -1, 128).max(axis=2)
    assert np.all((top >= 0x76) & (top <= 0x7E))
    _qdq_check(x, q, np.repeat(s.astype(np.float64), 128, axis=1))


def test_pow2_weight_invariants():
    w = workloads.dense(seed=2, M=128, N=256, K=384)["w"].float().numpy()
    q, s = quant.quant_128x128(w, scale="pow2")
    e = _exponent(s)
    amax = np.abs(w.astype(np.float64)).reshape(2, 128, 3, 128).max(axis=(1, 3))
    assert np.all(np.ldexp(amax, -e) <= 448.0) and np.all(np.ldexp(amax, -e) > 224.0)
    _qdq_check(w, q, np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1))


def test_pow2_against_the_microscaling_floor_rule():
    """Second derivation: the microscaling rule takes 2^(floor(log2 amax) - 8);
    the pages' no-clipping rule needs one power of two more exactly when amax
    exceeds 448 times that."""
    for x in INPUTS.values():
        _, s = quant.quant_1x128(x, scale="pow2")
        amax = np.abs(x.astype(np.float64)).reshape(x.shape[0], -1, 128).max(axis=2)
        ef = np.floor(np.log2(amax)) - 8
        want = ef + (amax > 448.0 * np.exp2(ef))
        assert np.array_equal(_exponent(s), want)


def test_pow2_scale_brackets_the_amax_scale():
    """amax/448 <= s < 2 * amax/448, so the fp32 amax scale s1 obeys s1 <= s <= 2 s1."""
    x = INPUTS["normal_outliers"]
    _, s1 = quant.quant_1x128(x)
    _, s2 = quant.quant_1x128(x, scale="pow2")
    assert np.all(s1 <= s2) and np.all(s2 <= 2 * s1)


@pytest.mark.parametrize("j", [-5, 3])
def test_pow2_equivariance(j):
    x = INPUTS["student_t"]
    q, s = quant.quant_1x128(x, scale="pow2")
    q2, s2 = quant.quant_1x128(np.ldexp(x, j).astype(np.float32), scale="pow2")
    assert np.array_equal(q, q2) and np.array_equal(s2, np.ldexp(s, j).astype(np.float32))
    qn, sn = quant.quant_1x128(-x, scale="pow2")
    assert np.array_equal(qn, q ^ 0x80) and np.array_equal(sn, s)


def test_pow2_zero_group():
    x = np.zeros((2, 256), np.float32)
    x[1, 128:] = 1.0
    x[0, 5] = -0.0
    q, s = quant.quant_1x128(x, scale="pow2")
    assert s[0].tolist() == [0.0, 0.0] and s[1, 0] == 0.0 and s[1, 1] == 2.0 ** -8
    assert q[0, 5] == 0x80 and np.all(q[1, 128:] == 0x38 + (8 << 3))  # 1.0 * 2^8 = 256 -> 0x78
