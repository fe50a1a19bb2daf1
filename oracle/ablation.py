"""Per-tensor against fine-grained scaling: the accuracy ablation.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

The innerforce notes' Figure 7(a) passage motivates the 1x128 / 128x128
grouping with the standard practice it replaces: one scale per tensor, set
by the tensor's largest magnitude, which leaves quantisation sensitive to
outliers -- a single large activation shrinks the scale for every other
element, pushing small values into the E4M3 subnormal range or to zero.
This module quantises the same inputs both ways and measures the damage.

* :func:`quant_per_tensor` -- the standard practice: s = fl32(amax/448) over
  the whole tensor, then the same fp32 steps and E4M3 cast as the group
  quantisers (oracle.quant).
* :func:`qdq_stats` -- element-wise quantise-dequantise error: relative
  error over the nonzero inputs (median, 99th percentile, mean), and the
  fractions of nonzero inputs that land below E4M3's normal range or at zero.
* :func:`gemm_error` -- relative Frobenius error of the fp64 product of the
  dequantised operands against the fp64 product of the unquantised ones.

* :func:`subnormal_fraction` -- the fraction of nonzero inputs whose code
  lies below E4M3's normal range (exponent field 0: zero or subnormal).

Parity (tests/test_oracle_ablation.py): the per-tensor quantiser is pinned by
a tensor that is one 1x128 tile (it quantises exactly as quant_1x128), 2^j
and sign equivariance and the amax element mapping to 0x7E.  Every function
here -- quant_per_tensor, dequant_per_tensor, qdq_stats, subnormal_fraction,
gemm_error, and the dequantisers of oracle.quant they are used with -- is
pinned by tests/golden/ablation_handworked.json: a 2x128 tensor with an
ordinary tile and a 64x outlier tile and a two-row weight, whose codes,
dequantised values, element-wise relative errors, statistics and GEMM errors
were worked out by hand as exact fractions.
"""

import numpy as np

from .e4m3 import E4M3_MAX, decode, encode
from .quant import dequant_128x128, dequant_1x128, quant_128x128, quant_1x128


def quant_per_tensor(x):
    """One scale for the whole tensor: returns (q uint8 like x, s fp32 scalar)."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("per-tensor quantisation: non-finite input is outside the contract")
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s = np.float32(amax / np.float32(E4M3_MAX))
    inv = np.float32(0) if s == 0 else np.float32(np.float32(1) / s)
    return encode(x * inv), s


def qdq_stats(x, deq):
    """Statistics of the quantise-dequantise error of the nonzero elements of x."""
    x = np.asarray(x, np.float64)
    deq = np.asarray(deq, np.float64)
    nz = x != 0
    rel = np.abs(deq[nz] - x[nz]) / np.abs(x[nz])
    return {
        "rel_median": float(np.median(rel)),
        "rel_p99": float(np.percentile(rel, 99)),
        "rel_mean": float(np.mean(rel)),
        "flushed_to_zero": float(np.mean(deq[nz] == 0)),
        "frac_nonzero": float(np.mean(nz)),
    }


def subnormal_fraction(q, x):
    """Fraction of nonzero inputs whose code is zero or subnormal (exponent field 0)."""
    q = np.asarray(q)
    nz = np.asarray(x) != 0
    return float(np.mean(((q & 0x78) == 0)[nz]))


def dequant_per_tensor(q, s):
    return decode(q) * np.float64(s)


def gemm_error(x, w, xa_deq, wb_deq):
    """||deq(X) deq(W)^T - X W^T||_F / ||X W^T||_F, all in fp64."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    ref = x @ w.T
    y = np.asarray(xa_deq, np.float64) @ np.asarray(wb_deq, np.float64).T
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def compare(x, w=None):
    """Per-tensor vs fine-grained on activations x (and the GEMM with w, if given)."""
    out = {}
    qa, sa = quant_1x128(x)
    qt, st = quant_per_tensor(x)
    fine = dequant_1x128(qa, sa)
    tens = dequant_per_tensor(qt, st)
    out["act_fine"] = {**qdq_stats(x, fine), "subnormal_or_zero": subnormal_fraction(qa, x)}
    out["act_tensor"] = {**qdq_stats(x, tens), "subnormal_or_zero": subnormal_fraction(qt, x)}
    if w is not None:
        qb, sb = quant_128x128(w)
        qw, sw = quant_per_tensor(w)
        wf = dequant_128x128(qb, sb)
        wt = dequant_per_tensor(qw, sw)
        out["weight_fine"] = qdq_stats(w, wf)
        out["weight_tensor"] = qdq_stats(w, wt)
        out["gemm_fine"] = gemm_error(x, w, fine, wf)
        out["gemm_tensor"] = gemm_error(x, w, tens, wt)
    return out


def main():
    """Print the ablation on the dense-projection inputs (X with 0.1% x100
    outliers, N(0, 0.02) weights; 512 of the 4096 rows) and on the Student-t
    activations of the quantiser workload (1024 of the 16384 rows)."""
    import json

    import workloads

    d = workloads.dense(M=512)
    res = {"dense_projection_512x7168x7168": compare(d["x"].float().numpy(), d["w"].float().numpy())}
    t = workloads.quant_act(M=1024)
    res["student_t_activations_1024x7168"] = compare(t.float().numpy())
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
