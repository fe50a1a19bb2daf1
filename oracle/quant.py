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

Parity: pinned.  tests/test_oracle_quant.py checks hand-worked tiles
(tests/golden/quant_tiles_handworked.json), the amax -> 0x7E invariant, the
quantise-dequantise error bound, power-of-two and sign equivariance, the
identity on E4M3-exact tiles, group locality, and the fp32 rounding of each
step against exact rational arithmetic.
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode

GROUP = 128


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


def _check_input(x):
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("quant: expected a 2-D array")
    x = x.astype(np.float32, copy=False)
    if not np.all(np.isfinite(x)):
        raise ValueError("quant: non-finite input is outside the contract")
    return x


def quant_1x128(x):
    """Quantise ``x`` [M, K] in 1x128 tiles along K.

    Returns ``(q, s)``: uint8 E4M3 codes [M, K] and fp32 scales
    [M, ceil(K/128)], where ``s[m, g]`` belongs to columns
    ``128*g .. 128*g+127`` of row ``m`` (a ragged last group covers the
    columns present).
    """
    x = _check_input(x)
    M, K = x.shape
    G = -(-K // GROUP)
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, G), dtype=np.float32)
    for g in range(G):
        cols = slice(g * GROUP, min(K, (g + 1) * GROUP))
        tile = x[:, cols]
        amax = np.max(np.abs(tile), axis=1) if tile.size else np.zeros(M, np.float32)
        sg, inv = _scale_and_inverse(amax)
        s[:, g] = sg
        q[:, cols] = encode(tile * inv[:, None])
    return q, s


def quant_128x128(w):
    """Quantise ``w`` [N, K] in 128x128 blocks.

    Returns ``(q, s)``: uint8 codes [N, K] and fp32 scales
    [ceil(N/128), ceil(K/128)], where ``s[i, j]`` belongs to rows
    ``128*i ..`` and columns ``128*j ..`` of ``w``.
    """
    w = _check_input(w)
    N, K = w.shape
    GN, GK = -(-N // GROUP), -(-K // GROUP)
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((GN, GK), dtype=np.float32)
    for i in range(GN):
        rows = slice(i * GROUP, min(N, (i + 1) * GROUP))
        for j in range(GK):
            cols = slice(j * GROUP, min(K, (j + 1) * GROUP))
            block = w[rows, cols]
            sb, inv = _scale_and_inverse(np.max(np.abs(block)))
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
