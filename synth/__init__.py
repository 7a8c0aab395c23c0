"""Seeded synthetic inputs for block-sparse FP8 attention prefill.

This package only draws random data and lays it out (quantised Q/K/V, paged
caches, page tables, block masks).  It holds none of the attention arithmetic,
and both the oracle-side tests and the GPU-side tests/benchmark use it.
"""
from .workloads import (CONFIGS, Problem, make_problem, WorkloadConfig, index_form,  # noqa: F401
                        topk_index_form, to_ntd, append_inputs)
from .decode import DECODE_CONFIGS, DecodeProblem, make_decode_problem  # noqa: F401,E402
