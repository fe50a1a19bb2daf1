"""Per-expert oracle work of the full-size MoE parity test, run in worker
processes (spawned, not forked, so they hold no GPU state and never touch
the GPU): each worker draws one expert's weight from the seeded generator,
quantises it with the oracle, and forms the oracle GEMM rows of that expert's
whole segment of routed rows."""

import hashlib

import numpy as np


def expert_reference(job):
    """job = (expert, oracle codes [r, K] and scales [r, K/128] of the rows of
    its segment).  Returns (expert, sha256 of the oracle weight codes, sha256
    of the oracle weight scales, fp64 oracle rows [r, N])."""
    e, ra, rsa = job
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import gemm, quant

    quant.CHUNK_ROWS = 1 << 30  # one thread per worker: the workers already fill the cores
    with threadpool_limits(limits=1):
        w = workloads.moe_expert_weight(e).float().numpy()
        qe, se = quant.quant_128x128(w)
        ref = gemm.block_gemm(ra, rsa, qe, se) if ra.shape[0] else np.zeros((0, qe.shape[0]))
    return e, hashlib.sha256(qe.tobytes()).hexdigest(), hashlib.sha256(se.tobytes()).hexdigest(), ref
