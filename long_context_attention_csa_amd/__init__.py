"""CSA/HCA hybrid attention forward for MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in libcsa_hip.so (include/csa_hip.h); this package is the
thin binding that marshals torch tensors into it.
"""
from .ops import (csa_compress, csa_quantize_rows, dense_attn_workspace_size,  # noqa: F401
                  dense_compressed_attn_fwd, hca_compress, indexer_topk, indexer_topk_workspace_size,
                  kernel_timer_read, kernel_timer_start, sparse_attn_fwd, sparse_attn_workspace_size)
