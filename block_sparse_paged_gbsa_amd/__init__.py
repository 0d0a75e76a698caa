"""Block-sparse flash attention over a paged KV cache for AMD MI355X (gfx950).

The computation lives in libgbsa.so (hand-written HIP kernels behind the C ABI of
include/gbsa.h); this package only marshals torch tensors into that ABI.
"""
from .api import (  # noqa: F401
    generic_block_sparse_attention,
    generic_block_sparse_attention_metadata,
    gbsa_check_params,
    gbsa_forward,
    gbsa_forward_tnd,
    gbsa_forward_ex,
    gbsa_forward_ex_noalloc,
    gbsa_validate,
    gbsa_metadata,
    gbsa_num_workers,
    gbsa_workspace_size,
    make_params,
    workspace_status,
)
from ._lib import GbsaError, GbsaParams  # noqa: F401
