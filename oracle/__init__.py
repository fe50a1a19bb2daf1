"""CPU oracle for the FP8 fine-grained quantization and block-scaled GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, tables or helpers with the HIP
library under ``fp8_fine_grained_amd/csrc``; the two meet only at the seeded
input generators (the top-level ``workloads`` module, which imports nothing
from the product package), which hold none of the
method's arithmetic.

Sources (the four web pages this work follows; each is cited by title and
section, never by line):

* "DeepSeek-V3 FP8 training notes" -- the innerforce.co.kr board post that
  paraphrases the DeepSeek-V3 report.  Its Figure 7(a) passage fixes the
  grouping (1x128 tiles per token for activations, 128x128 blocks for
  weights) and the scaling rule (the group's largest magnitude is mapped to
  the largest finite FP8 value).  Its accumulation passage fixes that the
  GEMM's partial sums are carried in FP32 and that dequantisation is folded
  into that higher-precision accumulation.
* The yunhecapital.com report, section 2.2.3 (mixed-precision framework for
  FP8 training): activations grouped 1x128 along the token dimension,
  weights 128x128 block-wise; MMA partials promoted to FP32 at a fixed
  interval.
* The tonho.wtf encyclopedia entry "DeepSeek-V3", section "como funciona":
  scale factors computed online, always the E4M3 format, partials promoted
  to FP32 every 128 elements.  Section "o que isso custou": gradient
  operands use 1x128 tiles (128x128 blocks on activation gradients diverged).
* The ruibaoantu.com mixed-precision article is about FP16/BF16 and is not
  used for anything here.

Modules:

* :mod:`oracle.e4m3`  -- OCP E4M3 ("E4M3FN") decode table and the saturating
  round-to-nearest-even encoder.
* :mod:`oracle.quant` -- 1x128 activation and 128x128 weight quantizers.
* :mod:`oracle.gemm`  -- fp64 GEMM on the dequantised operands, dense and
  grouped (per-expert row segments), plus row-sampled variants for checking
  full-size outputs.
* :mod:`oracle.ablation` -- per-tensor scaling (the practice the grouping
  replaces) against 1x128 / 128x128 groups: quantisation and GEMM error.

Every function here is plain numpy in the precision the method states
(fp32 for the scale/cast steps, where the result must be bit-exact) or fp64
(for the GEMM reference).  Parity status of each function is recorded in its
docstring; all are pinned by ``tests/test_oracle_*.py``.
"""

from . import e4m3, quant, gemm, ablation  # noqa: F401
