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
  * The FlashMLA FP8 sparse decoding article (gitcode.com, FlashMLA deep dive),
    sections "FP8 KVCache format" (the 656-byte token row), "Quant/dequant
    source" (1x128 tile scales amax/448, optionally rounded up to a power of
    two) and its description of the MQA decode step.

Contents
  e4m3      -- OCP FP8 E4M3FN codec written from the format definition.
  attention -- exact fp64 oracle, P-emulating oracle, brute-force oracle.
  schedule  -- task costs and the task order of the scheduling pre-pass.
  quantize  -- FP8 quantisation of Q and the K/V append into the paged cache.
  decode    -- FP8 sparse decode (MQA, 656-byte cache rows, top-k indices).

Every function is pinned by `tests/test_oracle_*.py`; the one part with no
independent pin ("parity unpinned") is agreement with the pages' own
implementations, whose outputs the pages do not print.
"""
from . import e4m3, attention, schedule, quantize, decode  # noqa: F401
