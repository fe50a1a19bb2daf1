"""fp8_fine_grained_amd: fine-grained FP8 (E4M3) quantisation and block-scaled
FP8 GEMM for AMD MI355X (gfx950).

The product is the C-ABI library ``libfp8fg.so`` (include/fp8fg.h) built from
``csrc/``; :mod:`fp8_fine_grained_amd.binding` calls it from Python with
torch tensors as device memory.  The seeded synthetic inputs come from the
top-level ``workloads`` module, outside this package.
"""

from .binding import (  # noqa: F401
    fp8_block_gemm,
    fp8_block_grouped_gemm,
    fp8_quant_act_1x128,
    fp8_quant_weight_128x128,
    lib,
)
