"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This package holds shapes (tensor tables of the models the pages train) and
seeded random generators.  It contains none of the compression method's
arithmetic: every number it produces is an *input* to both the HIP path and
the CPU oracle, which then compute independently from the same bytes.
"""

from .configs import (  # noqa: F401
    WORKLOADS,
    Workload,
    bert_large_tensors,
    gpt13b_tensors,
    segment_offsets,
)
