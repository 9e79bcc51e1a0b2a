"""CPU oracle of the ReSA decode hot path (test infrastructure only).

Importable by the tests, the package smoke check and the benchmark's
``cpu_baseline`` leg; never by the library.
"""

from .resa_oracle import *  # noqa: F401,F403
from .resa_oracle import (  # noqa: F401
    BLOCK, SCORE_MEAN_POOL, SCORE_SUM_HEADS, attend, block_descriptor, block_rows, dense,
    descriptors, memory_factor, num_blocks, rectify, scores, select, selection_count,
    touched_blocks,
)
