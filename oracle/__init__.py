"""CPU oracle for the weight-quantised GEMV/GEMM path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.
The product path (``gemm_wq_quantize_amd``) never imports it and has no CPU
fallback.

The oracle is written from the pages' text and shares no code with the HIP
path: the only common input is the seeded raw data of ``wq_inputs``.  It is
plain numpy: every integer step is exact, every floating result is carried in
float64 unless a step fixes its own precision (the quantisers round in float32
and store bf16 / fp16 exactly as the readings below state).

Pages cited (short names used in docstrings):
  * Paddle PR -- "[PHI] add int4 weight only quant kernel, add int4 weight
    only permute kernel" (PaddlePaddle/Paddle #64091)
  * Vulkan post -- "怎样在安卓端利用 Vulkan 编写 4-bit 专用算子：直接在 GPU
    上进行解量化与计算融合" (tbr8.org)
  * Helion issue -- "int4 gemm kernel" (pytorch/helion #508)
  * Ternary post -- "三值量化模型的无损压缩" (aduhtkjm.github.io)

Parity pins live in ``tests/test_oracle_*.py``.  Functions whose reading is
pinned only by invariants (not by a value printed on the pages) say
"parity unpinned" in their docstring: the int4 quantiser formula, the gfx950
nibble order, the ternary digit encoding and the PTQ1_1 bit positions and
codebook order (pinned by round trips, sizes and hand-worked bytes only).
"""
from . import fpformat, int4, ternary  # noqa: F401
