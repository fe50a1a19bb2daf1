"""OCP 8-bit floating point, E4M3 variant ("E4M3FN"): decode table and encoder.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

The pages fix the format: every FP8 tensor on the path is E4M3 (tonho.wtf
"DeepSeek-V3", section "como funciona").  The bit layout is that of the OCP
8-bit floating point specification's E4M3 format, which is what gfx950's FP8
instructions use:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 holds subnormals  m * 2^-9  (m = 0..7);
* exponent field e = 1..15 holds  (1 + m/8) * 2^(e-7);
* there is no infinity; the single pattern S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448 (code 0x7E).

The encoder is the saturating round-to-nearest-even cast that the
quantizers use: magnitudes are clamped to 448, then rounded to the nearest
point of the 127-value non-negative grid, ties going to the code whose
mantissa LSB is 0; the sign bit is copied from the input, so -0.0 and small
negatives that round to zero give 0x80.

Parity: pinned.  The decode table is checked against torch's
``float8_e4m3fn`` for all 254 finite codes; the encoder against torch's cast
(after clamping) on every grid midpoint and its neighbours plus random fp32
patterns, against brute-force nearest search, and against spec values
(tests/test_oracle_e4m3.py).
"""

import numpy as np

#: Largest finite E4M3 magnitude (code 0x7E).
E4M3_MAX = 448.0

#: Number of non-negative finite codes (0x00 .. 0x7E).
_N_FINITE = 127


def _decode_one(code):
    """Value of one E4M3 code (0..255) from its bit fields, as a Python float."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


#: fp64 value of every code 0..255 (NaN at 0x7F and 0xFF).
DECODE_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)

# Non-negative finite grid, strictly increasing: GRID[c] is the value of code c.
_GRID = DECODE_TABLE[:_N_FINITE].copy()
# Midpoints between neighbouring grid values.  All grid values are multiples
# of 2^-10 below 2^9, so the midpoints are exact in fp64.
_MIDS = (_GRID[:-1] + _GRID[1:]) * 0.5


def decode(codes):
    """fp64 values of an array of E4M3 codes (uint8)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y):
    """Saturating RNE cast of fp32 values to E4M3 codes (uint8).

    ``y`` must be finite (NaN/Inf are outside the method's contract).
    """
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("E4M3 encode: non-finite input is outside the contract")
    a = np.minimum(np.abs(y).astype(np.float64), E4M3_MAX)
    # i = number of midpoints strictly below a: the nearest grid point is code
    # i unless a sits exactly on midpoint i, a tie between codes i and i+1.
    i = np.searchsorted(_MIDS, a, side="left")
    tie = np.zeros(a.shape, dtype=bool)
    inside = i < _MIDS.size
    tie[inside] = a[inside] == _MIDS[i[inside]]
    code = np.where(tie & (i % 2 == 1), i + 1, i).astype(np.uint8)
    return code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))
