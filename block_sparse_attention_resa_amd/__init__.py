"""ReSA decode hot path on MI355X: Python face of libresa.

The library (libresa.so, built from csrc/ by ``python -m
block_sparse_attention_resa_amd.build``) exports the C ABI declared in
include/resa.h.  This package only marshals torch tensors into those calls.
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    OP_DENSE_DECODE,
    OP_DENSE_RECTIFY,
    OP_SCORE_SELECT,
    OP_SPARSE_DECODE,
    OP_SPARSE_STEP,
    RESA_BF16,
    RESA_F32,
    RESA_SCORE_MEAN_POOL,
    RESA_SCORE_SUM_HEADS,
    Config,
    PagedKV,
    ResaError,
    abi_version,
    alloc_workspace,
    build_descriptors,
    dense_decode,
    dense_rectify,
    load_library,
    num_splits,
    score_select,
    selection_count,
    sparse_decode,
    sparse_decode_noalloc,
    sparse_step,
    NOALLOC_SCRATCH_BYTES,
    workspace_bytes,
)
