"""Fine-grained FP8 quantizers: 1x128 activation tiles and 128x128 weight blocks.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

What is computed, and where the pages say it:

* Grouping -- activations per 1x128 tile (one token, 128 consecutive
  channels), weights per 128x128 block (128 output x 128 input channels):
  DeepSeek-V3 FP8 training notes (innerforce.co.kr), Figure 7(a) passage;
  yunhecapital.com report section 2.2.3; tonho.wtf "DeepSeek-V3",
  "como funciona".
* Scale -- each group's largest magnitude is mapped onto the largest finite
  FP8 value: innerforce notes, Figure 7(a) passage (the practice it refines
  maps the whole tensor's amax; the method applies the same rule per group).
  The largest finite E4M3 value is 448, so the group scale is amax / 448.
* Online, E4M3 -- the factor is computed from the data at quantisation time
  and the format is always E4M3: tonho.wtf "DeepSeek-V3", "como funciona".
* Gradient operands use 1x128 tiles along the contraction axis (the token
  axis of the weight-gradient GEMM): tonho.wtf "DeepSeek-V3",
  "o que isso custou".  :func:`quant_1x128_along_rows` is that case.

Per group, in IEEE fp32 with round-to-nearest-even and each operation
rounded on its own (readings where the pages are silent):

    amax = max |x_i|                       (exact)
    s    = fl32(amax / 448)                (true division)
    inv  = 0 if s == 0 else fl32(1 / s)
    y_i  = fl32(x_i * inv)                 (one multiply, not x_i / s)
    q_i  = E4M3 saturating RNE cast of y_i (oracle.e4m3.encode)

An all-zero group gets s = 0 and codes 0x00/0x80 (sign kept), so its
dequantised value dec(q) * s is exactly zero.  Non-finite inputs and groups
whose scale would be subnormal (0 < amax < 448 * 2^-126) are outside the
contract and raise ValueError.

Power-of-two scales (the ``*_pow2`` functions).  The innerforce notes'
Figure 7(a) passage calls the grouping consistent with microscaling formats,
and the tonho.wtf entry's "o que isso custou" wish list asks for an MMA that
applies per-group scales itself.  Microscaling scales are powers of two (the
E8M0 format), which is what gfx950's scaled matrix-core instructions take.
The pages fix neither that format nor its rounding; the reading taken keeps
the pages' scaling rule (the group's amax lands on or below 448, nothing is
clipped) with the scale restricted to powers of two:

    s    = 2^e, e the smallest integer with amax <= 448 * 2^e
           (so 224 < amax / s <= 448)
    inv  = 2^-e                              (exact)
    y_i  = fl32(x_i * inv),  q_i = E4M3 RNE cast of y_i (as above)

An all-zero group again gets s = 0 and inv = 0.  Groups whose e or -e falls
outside fp32's normal exponent range are outside the contract.

Parity: pinned.  tests/test_oracle_quant.py checks hand-worked tiles
(tests/golden/quant_tiles_handworked.json), the amax -> 0x7E invariant, the
quantise-dequantise error bound, power-of-two and sign equivariance, the
identity on E4M3-exact tiles, group locality, and the fp32 rounding of each
step against exact rational arithmetic.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .e4m3 import E4M3_MAX, encode

GROUP = 128
#: Rows per work item when a quantiser splits its input over threads (a
#: multiple of 128, so a chunk holds whole 128x128 weight blocks).
CHUNK_ROWS = 512


def threads():
    """Host threads the oracle uses: the cores this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _by_row_chunks(one, x, scale, group_rows):
    """Run the quantiser ``one`` on consecutive row chunks of ``x`` in threads.

    Groups never straddle a chunk (chunks are whole multiples of the group
    height), so the result is the same as one call over all rows: the chunks
    only divide the work.  numpy releases the interpreter lock inside its
    array operations, so the threads run in parallel."""
    assert CHUNK_ROWS % group_rows == 0
    n = x.shape[0]
    nt = threads()
    if nt == 1 or n <= CHUNK_ROWS:
        return one(x, scale)
    starts = list(range(0, n, CHUNK_ROWS))
    with ThreadPoolExecutor(min(nt, len(starts))) as ex:
        parts = list(ex.map(lambda r0: one(x[r0:r0 + CHUNK_ROWS], scale), starts))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _scale_and_inverse(amax):
    """fp32 scale amax/448 and its fp32 reciprocal (0 for an all-zero group)."""
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / np.float32(E4M3_MAX)
    inv = np.zeros_like(s)
    with np.errstate(over="ignore"):
        np.divide(np.float32(1.0), s, out=inv, where=(s != 0))
    if np.any((s != 0) & (s < np.finfo(np.float32).tiny)):
        raise ValueError("quant: group amax below 448*2^-126 is outside the contract")
    return s.astype(np.float32), inv.astype(np.float32)


def _pow2_scale_and_inverse(amax):
    """Power-of-two scale 2^e (smallest e with amax <= 448 * 2^e) and 2^-e."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    nz = a != 0
    # a = f * 2^E with f in [0.5, 1): a * 2^-(E-9) = f * 2^9 lies in [256, 512);
    # it is within 448 unless f > 7/8, and one power of two more always is.
    _, E = np.frexp(a)
    e = E - 9
    e = np.where(np.ldexp(a, -e) > E4M3_MAX, e + 1, e)
    if np.any(nz & ((e < -126) | (e > 126))):
        raise ValueError("quant: power-of-two scale outside fp32's normal range is outside the contract")
    s = np.where(nz, np.ldexp(1.0, e), 0.0).astype(np.float32)
    inv = np.where(nz, np.ldexp(1.0, -e), 0.0).astype(np.float32)
    return s, inv


_SCALES = {"amax": _scale_and_inverse, "pow2": _pow2_scale_and_inverse}


def _check_input(x):
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("quant: expected a 2-D array")
    x = x.astype(np.float32, copy=False)
    if not np.all(np.isfinite(x)):
        raise ValueError("quant: non-finite input is outside the contract")
    return x


def quant_1x128(x, scale="amax"):
    """Quantise ``x`` [M, K] in 1x128 tiles along K.

    Returns ``(q, s)``: uint8 E4M3 codes [M, K] and fp32 scales
    [M, ceil(K/128)], where ``s[m, g]`` belongs to columns
    ``128*g .. 128*g+127`` of row ``m`` (a ragged last group covers the
    columns present).  ``scale="pow2"`` takes power-of-two scales.
    Large inputs are split into row chunks quantised in parallel threads.
    """
    return _by_row_chunks(_quant_1x128, _check_input(x), scale, 1)


def _quant_1x128(x, scale):
    scale_and_inverse = _SCALES[scale]
    M, K = x.shape
    G = -(-K // GROUP)
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, G), dtype=np.float32)
    for g in range(G):
        cols = slice(g * GROUP, min(K, (g + 1) * GROUP))
        tile = x[:, cols]
        amax = np.max(np.abs(tile), axis=1) if tile.size else np.zeros(M, np.float32)
        sg, inv = scale_and_inverse(amax)
        s[:, g] = sg
        q[:, cols] = encode(tile * inv[:, None])
    return q, s


def quant_128x128(w, scale="amax"):
    """Quantise ``w`` [N, K] in 128x128 blocks.

    Returns ``(q, s)``: uint8 codes [N, K] and fp32 scales
    [ceil(N/128), ceil(K/128)], where ``s[i, j]`` belongs to rows
    ``128*i ..`` and columns ``128*j ..`` of ``w``.  ``scale="pow2"`` takes
    power-of-two scales.  Large inputs are split into chunks of whole block
    rows quantised in parallel threads.
    """
    return _by_row_chunks(_quant_128x128, _check_input(w), scale, GROUP)


def _quant_128x128(w, scale):
    scale_and_inverse = _SCALES[scale]
    N, K = w.shape
    GN, GK = -(-N // GROUP), -(-K // GROUP)
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((GN, GK), dtype=np.float32)
    for i in range(GN):
        rows = slice(i * GROUP, min(N, (i + 1) * GROUP))
        for j in range(GK):
            cols = slice(j * GROUP, min(K, (j + 1) * GROUP))
            block = w[rows, cols]
            sb, inv = scale_and_inverse(np.max(np.abs(block)))
            s[i, j] = sb
            q[rows, cols] = encode(block * inv)
    return q, s


def quant_1x128_along_rows(x):
    """Quantise ``x`` [T, C] in 1x128 tiles running down each column.

    This is the gradient-operand case: the groups lie along the token axis T,
    which is the contraction axis of the weight-gradient GEMM.  Returns the
    codes already transposed, ``q`` [C, T], with scales [C, ceil(T/128)], so
    that the result is exactly ``quant_1x128(x.T)``.
    """
    x = _check_input(x)
    return quant_1x128(np.ascontiguousarray(x.T))


def dequant_1x128(q, s):
    """fp64 values dec(q[m,k]) * s[m, k//128] of a 1x128-quantised matrix."""
    from .e4m3 import decode

    q = np.asarray(q)
    K = q.shape[1]
    return decode(q) * np.repeat(np.asarray(s, np.float64), GROUP, axis=1)[:, :K]


def dequant_128x128(q, s):
    """fp64 values dec(q[n,k]) * s[n//128, k//128] of a 128x128-quantised matrix."""
    from .e4m3 import decode

    q = np.asarray(q)
    N, K = q.shape
    se = np.repeat(np.repeat(np.asarray(s, np.float64), GROUP, axis=0), GROUP, axis=1)
    return decode(q) * se[:N, :K]
