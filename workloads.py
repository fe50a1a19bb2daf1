"""Seeded synthetic inputs shaped like the DeepSeek-V3 FP8 workloads.

This module draws random numbers and arranges them; it holds none of the
quantisation or GEMM arithmetic.  Both the HIP path (tests, benchmark) and
the CPU oracle take their inputs from here, which is the only thing they
share.

Shapes follow the model the pages describe: hidden size 7168, 256 routed
experts with 8 active per token (tonho.wtf "DeepSeek-V3", "como funciona";
yunhecapital.com report section 2.2.2).  The pages name no dataset; every
input is synthetic.  Recipes (numpy ``default_rng``, fp32 draws, cast to
bfloat16 with round-to-nearest-even where the workload is bf16):

* ``tiny``      X fp32 [128,256] ~ N(0,1) with 1% of entries x50;
                W fp32 [128,256] ~ N(0, 0.02).
* ``dense``     X bf16 [4096,7168] ~ N(0,1) with 0.1% of entries x100;
                W bf16 [7168,7168] ~ N(0, 0.02).
* ``quant``     activation bf16 [16384,7168] Student-t (nu=3, unscaled);
                weight bf16 [7168,18432] ~ N(0, 0.02).
* ``moe``       tokens bf16 [8192,7168] ~ N(0,1); affinity logits
                [8192,256] ~ N(0,1) plus a per-expert bias ~ U(-0.01,0.01);
                each token goes to the 8 experts of largest logit+bias (ties
                to the lower expert id); rows sorted by (expert, token) give
                65536 permuted rows and 257 segment offsets; expert weights
                bf16 [2048,7168] ~ N(0, 0.02), drawn per expert on demand.
* ``wgrad``     dY bf16 [16384,7168] ~ N(0, 1e-3); X bf16 [16384,7168] ~ N(0,1).
* ``dgrad``     dY bf16 [4096,7168] ~ N(0, 1e-3); W bf16 [7168,7168] ~ N(0, 0.02)
                (the data gradient dX = dY W of the dense projection).

N(mu, sigma) names the standard deviation.  Outliers: exactly
floor(p * numel) positions drawn without replacement, multiplied by the
factor.  Every generator takes its sizes as arguments so tests can draw
smaller inputs of the same distribution.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

_CHUNK_ROWS = 512  # rows per independently seeded chunk (fixed: results never depend on thread count)


def _threads():
    try:
        import os

        return max(1, min(16, len(os.sched_getaffinity(0))))
    except Exception:  # pragma: no cover
        return 4


def _draw(shape, seed, tag, kind, **kw):
    """fp32 array of ``shape`` from chunk-seeded generators (deterministic)."""
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.float32)
    starts = list(range(0, rows, _CHUNK_ROWS))

    def fill(i):
        r0 = starts[i]
        r1 = min(rows, r0 + _CHUNK_ROWS)
        rng = np.random.default_rng([seed, tag, i])
        n = (r1 - r0, cols)
        if kind == "normal":
            v = rng.standard_normal(n, dtype=np.float32)
            if kw.get("std", 1.0) != 1.0:
                v *= np.float32(kw["std"])
        elif kind == "student_t":
            v = rng.standard_t(kw["nu"], size=n).astype(np.float32)
        elif kind == "uniform":
            v = rng.uniform(kw["lo"], kw["hi"], size=n).astype(np.float32)
        else:  # pragma: no cover
            raise ValueError(kind)
        out[r0:r1] = v

    if len(starts) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(starts))))
    else:
        fill(0)
    return out


def _outliers(x, frac, factor, seed, tag):
    k = int(np.floor(frac * x.size))
    if k:
        rng = np.random.default_rng([seed, tag, 999_999])
        idx = rng.choice(x.size, size=k, replace=False)
        flat = x.reshape(-1)
        flat[idx] *= np.float32(factor)
    return x


def to_bf16(a):
    """torch CPU bfloat16 tensor from an fp32 array (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def tiny(seed=1, M=128, N=128, K=256):
    """Tiny case: fp32 X [M,K] with 1% x50 outliers, fp32 W [N,K] ~ N(0,0.02)."""
    x = _outliers(_draw((M, K), seed, 1, "normal"), 0.01, 50.0, seed, 1)
    w = _draw((N, K), seed, 2, "normal", std=0.02)
    return {"x": torch.from_numpy(x), "w": torch.from_numpy(w)}


def dense(seed=2, M=4096, N=7168, K=7168):
    """Dense projection: bf16 X [M,K] with 0.1% x100 outliers, bf16 W [N,K] ~ N(0,0.02)."""
    x = _outliers(_draw((M, K), seed, 1, "normal"), 0.001, 100.0, seed, 1)
    w = _draw((N, K), seed, 2, "normal", std=0.02)
    return {"x": to_bf16(x), "w": to_bf16(w)}


def quant_act(seed=3, M=16384, K=7168):
    """Quantizer bandwidth, activation: bf16 [M,K] Student-t with nu=3."""
    return to_bf16(_draw((M, K), seed, 1, "student_t", nu=3.0))


def quant_weight(seed=3, N=7168, K=18432):
    """Quantizer bandwidth, weight: bf16 [N,K] ~ N(0,0.02)."""
    return to_bf16(_draw((N, K), seed, 2, "normal", std=0.02))


def route_topk(logits, bias, topk):
    """Top-k experts per token on logits+bias; returns (perm, offsets, experts).

    ``perm[r]`` is the token of permuted row r, rows sorted by (expert, token);
    ``offsets`` [E+1] delimit each expert's rows.
    """
    T, E = logits.shape
    score = logits.astype(np.float32) + bias.astype(np.float32)[None, :]
    # stable sort of -score: ties keep the lower expert id first
    order = np.argsort(-score, axis=1, kind="stable")[:, :topk]
    tok = np.repeat(np.arange(T, dtype=np.int64), topk)
    exp = order.reshape(-1).astype(np.int64)
    key = np.lexsort((tok, exp))
    perm = tok[key]
    counts = np.bincount(exp, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return perm, offsets, exp[key]


def moe_routing(seed=4, T=8192, E=256, topk=8):
    """Affinity logits ~ N(0,1) + bias ~ U(-0.01,0.01), top-k routing."""
    logits = _draw((T, E), seed, 1, "normal")
    bias = _draw((1, E), seed, 2, "uniform", lo=-0.01, hi=0.01)[0]
    perm, offsets, experts = route_topk(logits, bias, topk)
    return {"perm": perm, "offsets": offsets, "experts": experts}


def moe_tokens(seed=4, T=8192, H=7168):
    """Token activations bf16 [T,H] ~ N(0,1)."""
    return to_bf16(_draw((T, H), seed, 3, "normal"))


def moe_expert_weight(g, seed=4, N=2048, K=7168):
    """Expert g's up-projection weight bf16 [N,K] ~ N(0,0.02)."""
    return to_bf16(_draw((N, K), seed, 100 + int(g), "normal", std=0.02))


def wgrad(seed=5, T=16384, C=7168, Cin=None):
    """Weight-gradient operands: dY bf16 [T,C] ~ N(0,1e-3), X bf16 [T,Cin] ~ N(0,1)."""
    Cin = C if Cin is None else Cin
    dy = _draw((T, C), seed, 1, "normal", std=1e-3)
    x = _draw((T, Cin), seed, 2, "normal")
    return {"dy": to_bf16(dy), "x": to_bf16(x)}


def dgrad(seed=6, M=4096, N=7168, K=7168):
    """Data-gradient operands: dY bf16 [M,N] ~ N(0,1e-3), W bf16 [N,K] ~ N(0,0.02)."""
    dy = _draw((M, N), seed, 1, "normal", std=1e-3)
    w = _draw((N, K), seed, 2, "normal", std=0.02)
    return {"dy": to_bf16(dy), "w": to_bf16(w)}


def skewed_offsets(M_total, G, big_rows, n_empty, seed=7):
    """Segment offsets with one expert of ``big_rows`` rows and ``n_empty`` empty experts."""
    rng = np.random.default_rng([seed, 77])
    counts = np.zeros(G, dtype=np.int64)
    empties = set(rng.choice(np.arange(1, G), size=n_empty, replace=False).tolist())
    counts[0] = big_rows
    rest = [g for g in range(1, G) if g not in empties]
    left = M_total - big_rows
    if rest:
        cut = np.sort(rng.integers(0, left + 1, size=len(rest) - 1))
        counts[rest] = np.diff(np.concatenate([[0], cut, [left]]))
    offsets = np.zeros(G + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return offsets


def moe_expert_weights(experts, seed=4, N=2048, K=7168):
    """Stacked bf16 [len(experts), N, K] of the given experts' weights (threaded over experts)."""
    experts = list(experts)
    out = torch.empty((len(experts), N, K), dtype=torch.bfloat16)

    def one(i):
        g = experts[i]
        rng_rows = []
        for c, r0 in enumerate(range(0, N, _CHUNK_ROWS)):
            r1 = min(N, r0 + _CHUNK_ROWS)
            rng = np.random.default_rng([seed, 100 + int(g), c])
            v = rng.standard_normal((r1 - r0, K), dtype=np.float32)
            v *= np.float32(0.02)
            rng_rows.append(v)
        out[i] = to_bf16(np.concatenate(rng_rows))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(len(experts))))
    return out
