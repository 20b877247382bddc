"""CPU oracle for fine-grained FP8 quantisation and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
CPU statement of what the GPU path computes.  Only ``tests/``, the smoke
check in ``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  The GPU library never calls it, and it imports nothing from
the GPU package: the two share no code.

Sources (web pages on DeepSeek-V3's FP8 training; they have no section
numbers, so a passage is located by page and paragraph):

  P1  "DeepSeek core readings" notes page (why-be.why-be.co.kr)
  P2  Q&A board page (xn--9g3bo1gtkw0l8ubf92bgle.kr)
  P3  "How I Improved My Deepseek In In The Future" (youlimart.com)
  P4  "How Google Is Changing How We Method Deepseek" (xn--jj0bz6z98ct0a29q.com)
  P5  cluster / communication notes page (cameseeing.com)

  * 1x128 activation tiles and 128x128 weight blocks: P1, paragraph 1.
  * scale from the max-abs value, mapped onto the largest FP8 value, and
    derived online: P2 paragraphs 3-4, P4 paragraph 1.
  * per-group scales along K, multiplied in as dequantisation, with FP32
    accumulation: P2 paragraph 3, P4 paragraph 4, P1 paragraph 4.
  * normalisation fused with the FP8 cast, norm kept in higher precision:
    P3 paragraph 3, P2 paragraph 1.
  * activations quantised to FP8 before they are dispatched to the MoE
    experts: P2 paragraph 4; 8 routed experts per token: P3 paragraph 4.

The pages fix neither the FP8 format nor the constant; the workload
definition fixes E4M3 and ``scale = amax / 448``.  Every other open point is
a stated reading, listed in the module that takes it.

Precision: quantisation is exact-spec IEEE binary32 (NumPy float32 on x86,
no flush-to-zero), so it has one correct answer per input.  The GEMM is its
definition evaluated in float64.

The per-tensor-scaling ablation (``oracle.ablation``, run as ``python -m
oracle.ablation``) quantises the same operands with one scale per tensor and
reports both products' errors against the unquantised BF16 product; it is a
reported diagnostic of the pages' outlier claim [P2 paragraph 3, P4
paragraph 3], not a gate.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, exhaustive enumeration or library
routines.  The summation order of the fused RMSNorm
(``oracle.quant.sum_squares_r64``) is a reading the pages do not fix; it is
pinned by crafted rows whose hand-derived binary32 sums differ from those of
a sequential sum, contiguous per-partial vectors, a reversed butterfly and a
fused multiply-add accumulation.
"""
from .e4m3 import (  # noqa: F401
    E4M3_MAX,
    FLT_MAX,
    e4m3_decode,
    e4m3_decode_table,
    e4m3_encode,
)
from .quant import (  # noqa: F401
    f32_from_bf16,
    fused_rmsnorm_quant,
    quant_act_1x128,
    quant_w_128x128,
    rmsnorm_r64,
    sum_squares_r64,
)
from .gemm import (  # noqa: F401
    bf16_round_f64,
    dequant_act,
    dequant_w,
    gemm_gate,
    gemm_ref,
    grouped_gemm_ref,
)
from .dispatch import (  # noqa: F401
    dispatch_ref,
    quant_dispatch_e8m0_ref,
    quant_dispatch_ref,
)
from .e8m0 import (  # noqa: F401
    e8m0_decode,
    e8m0_exponent,
    fused_rmsnorm_quant_e8m0,
    gemm_e8m0_ref,
    grouped_gemm_e8m0_ref,
    quant_act_1x128_e8m0,
    quant_w_128x128_e8m0,
)
