"""CSA/HCA hybrid attention forward for MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in libcsa_hip.so (include/csa_hip.h); this package is the
thin binding that marshals torch tensors into it.
"""
from .ops import (csa_append_state, csa_compress, csa_compress_append,  # noqa: F401
                  csa_quantize_rows, dense_attn_bwd_workspace_size, dense_attn_workspace_size,
                  dense_compressed_attn_bwd, dense_compressed_attn_fwd, hca_append_state,
                  hca_compress, hca_compress_append, indexer_scores, indexer_topk, indexer_topk_workspace_size,
                  kernel_timer_read, kernel_timer_start, sparse_attn_bwd,
                  sparse_attn_bwd_workspace_size, sparse_attn_fwd, sparse_attn_fwd_noalloc,
                  sparse_attn_noalloc_scratch_bytes, sparse_attn_workspace_size,
                  window_append, state_checkpoint, state_restore, ring_fill,
                  linear_bf16, grouped_out_proj, query_proj_shared,
                  grouped_out_proj_workspace_size, query_proj_shared_workspace_size, kv_proj)
