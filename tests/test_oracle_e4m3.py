"""Pins for oracle.e4m3 against the OCP E4M3 format definition, torch's
independent float8_e4m3fn codec, brute-force nearest search and fixed values."""

import math

import numpy as np
import torch

from oracle import e4m3
from tests.exact import e4m3_values_torch


def test_decode_table_matches_torch_for_every_code():
    ref = e4m3_values_torch()
    for c in range(256):
        v = e4m3.DECODE_TABLE[c]
        if c in (0x7F, 0xFF):
            assert math.isnan(v) and math.isnan(ref[c])
            continue
        assert v == ref[c], hex(c)
        assert math.copysign(1.0, v) == math.copysign(1.0, ref[c]), hex(c)


def test_format_constants():
    t = e4m3.DECODE_TABLE
    assert t[0x7E] == 448.0 == e4m3.E4M3_MAX
    assert t[0x08] == 2.0 ** -6  # smallest normal
    assert t[0x01] == 2.0 ** -9  # smallest subnormal
    assert t[0x38] == 1.0
    finite = t[:0x7F]
    assert np.all(np.diff(finite) > 0), "non-negative codes must be strictly increasing"


def test_spec_values():
    cases = [
        (448.0, 0x7E),
        (447.0, 0x7E),
        (464.0, 0x7E),  # beyond the grid: saturate, never NaN
        (1e30, 0x7E),
        (2.0 ** -6, 0x08),
        (2.0 ** -9, 0x01),
        (2.0 ** -10, 0x00),  # tie between 0 and 2^-9 -> even code 0
        (1.5 * 2.0 ** -10, 0x01),
        (7.5 * 2.0 ** -9, 0x08),  # tie across the subnormal/normal seam -> even code 0x08
        (1.0, 0x38),
        (1.0625, 0x38),  # tie between 0x38 and 0x39 -> 0x38
        (1.1875, 0x3A),  # tie between 0x39 and 0x3A -> 0x3A
        (0.0, 0x00),
        (-0.0, 0x80),
        (-1e-30, 0x80),  # rounds to zero, sign kept
        (-448.0, 0xFE),
        (-1e30, 0xFE),
        (240.0, 0x77),
        (416.0, 0x7D),
        (432.0, 0x7E),  # tie between 416 (0x7D) and 448 (0x7E) -> even 0x7E
    ]
    got = e4m3.encode(np.array([c[0] for c in cases], dtype=np.float32))
    for (x, want), g in zip(cases, got):
        assert g == want, (x, hex(g), hex(want))


def _probe_points():
    grid = e4m3.DECODE_TABLE[:0x7F].astype(np.float32)
    mids = ((grid[:-1].astype(np.float64) + grid[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (grid[:-1].astype(np.float64) + grid[1:]) / 2)
    pts = [grid, mids]
    for p in (grid, mids):
        up, dn = p.copy(), p.copy()
        for _ in range(3):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
            pts += [up, dn]
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 0x43FA0000, size=400_000, dtype=np.uint32)  # 0 .. 500
    pts.append(bits.view(np.float32))
    pts.append(np.float32(2.0) ** np.arange(-149, 10, dtype=np.float32))
    x = np.concatenate(pts).astype(np.float32)
    x = x[np.isfinite(x)]
    return np.concatenate([x, -x])


def test_encode_matches_torch_cast_after_clamp():
    x = _probe_points()
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_encode_brute_force_nearest():
    rng = np.random.default_rng(12)
    x = np.concatenate([
        rng.integers(0, 0x43E00000, size=30_000, dtype=np.uint32).view(np.float32),
        (e4m3.DECODE_TABLE[:0x7F][:-1] + e4m3.DECODE_TABLE[:0x7F][1:]).astype(np.float32) / 2,
    ])
    grid = [e4m3.DECODE_TABLE[c] for c in range(0x7F)]
    got = e4m3.encode(x)
    for xi, gi in zip(x.tolist(), got.tolist()):
        d = [abs(xi - v) for v in grid]
        best = min(d)
        cands = [c for c in range(0x7F) if d[c] == best]
        want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        assert gi == want, (xi, gi, want)


def test_encode_monotone_unit_steps_over_dense_sweep():
    bits = np.arange(0, 0x43E00001, 97, dtype=np.uint32)
    codes = e4m3.encode(bits.view(np.float32)).astype(np.int64)
    step = np.diff(codes)
    assert step.min() >= 0 and step.max() <= 1
    assert codes[0] == 0 and codes[-1] == 0x7E


def test_encode_never_nan_code():
    x = _probe_points() * np.float32(3.0)
    c = e4m3.encode(x)
    assert not np.any((c & 0x7F) == 0x7F)


def test_encode_exhaustive_against_torch_thresholds():
    """Every non-negative fp32 up to 464 (and its negation), through torch's codec.

    torch's codes over all 1.14e9 bit patterns in [0, 464] form a staircase with
    unit steps; the oracle's encoder is monotone by construction (a search over
    increasing midpoints), so it equals torch on the whole range exactly when it
    switches codes at the same 126 fp32 values.  Beyond 464 torch gives NaN and
    the oracle saturates (checked in test_spec_values)."""
    top = int(np.float32(464.0).view(np.uint32))
    chunk = 1 << 27
    first = {}  # code -> first bit pattern carrying it
    prev_code = None
    for lo in range(0, top + 1, chunk):
        hi = min(lo + chunk, top + 1)
        bits = torch.arange(lo, hi, dtype=torch.int32)
        for sign in (0, 1):
            x = bits.view(torch.float32)
            if sign:
                x = -x
            c = x.to(torch.float8_e4m3fn).view(torch.uint8)
            if sign:
                assert bool(torch.all((c & 0x80) == 0x80)), "negative inputs keep the sign bit"
                c = c & 0x7F
                assert bool(torch.all(c == pos)), "torch's codec is sign-symmetric"
                continue
            pos = c
            step = c[1:].to(torch.int16) - c[:-1].to(torch.int16)
            assert int(step.min()) >= 0 and int(step.max()) <= 1, "unit staircase"
            if prev_code is not None:
                assert 0 <= int(c[0]) - prev_code <= 1
                if int(c[0]) != prev_code:
                    first[int(c[0])] = lo
            else:
                assert int(c[0]) == 0
            for k in torch.nonzero(step).flatten().tolist():
                first[int(c[k + 1])] = lo + k + 1
            prev_code = int(c[-1])
    assert sorted(first) == list(range(1, 0x7F)), "every code 1 .. 0x7E is reached"
    thr = np.array([first[c] for c in range(1, 0x7F)], dtype=np.uint32)
    below = (thr - 1).view(np.float32)
    at = thr.view(np.float32)
    codes = np.arange(1, 0x7F, dtype=np.uint8)
    assert np.array_equal(e4m3.encode(at), codes)
    assert np.array_equal(e4m3.encode(below), codes - 1)
    assert np.array_equal(e4m3.encode(-at), codes | 0x80)
    assert np.array_equal(e4m3.encode(-below), (codes - 1) | 0x80)
