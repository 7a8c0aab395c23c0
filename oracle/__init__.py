"""CPU oracle for block-sparse FP8 attention prefill over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package.  The
GPU library never calls it, and it shares no code with the GPU library.

Sources (cited by page title and section throughout):
  * "Quant Block Sparse Attention" (CANNBotDSL sample, gitcode.com/cann/cannbot-dsl),
    sections "Operator introduction" (the attention formula and the feature /
    constraint table), "Key parameters", "Sparse indices & PA page table" and
    "Precision test".
  * The hpc-ops block-sparse FP8 attention article (hotelren.com/news/5676318),
    sections "Block-sparse scheduling", "Active tile list",
    "FP8 Tensor Core compute: fixed P-scale quantisation" and "Quick start".

Contents
  e4m3      -- OCP FP8 E4M3FN codec written from the format definition.
  attention -- exact fp64 oracle, P-emulating oracle, brute-force oracle.
  schedule  -- task costs and the task order of the scheduling pre-pass.

Every function is pinned by `tests/test_oracle_*.py`; the one part with no
independent pin ("parity unpinned") is agreement with the pages' own
implementations, whose outputs the pages do not print.
"""
from . import e4m3, attention, schedule  # noqa: F401
