"""Seeded synthetic inputs for the ReSA decode hot path.

This package produces inputs only: queries, keys, values, the paged layout the
library consumes and the logical per-request arrays the CPU oracle consumes.
It holds none of the method's arithmetic (no descriptors, scores, selection or
attention); both the HIP path and the oracle are fed from here.
"""

from .workloads import (  # noqa: F401
    BLOCK,
    WORKLOADS,
    WorkloadSpec,
    LayerInputs,
    Paged,
    make_layer,
    make_paged,
    make_append_rows,
    make_rectify_inputs,
    paged_to_logical,
    write_rows,
    num_blocks,
    round_bf16,
)
