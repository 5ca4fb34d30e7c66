"""MI355X (gfx950) compressed sparse attention hot path.

The work happens in ``libcsa.so`` (hand-written HIP kernels behind the C ABI
of ``include/csa.h``); this package only loads it and marshals arguments.
There is no CPU or PyTorch fallback: if the library is missing, ``load()``
raises.
"""
from ._abi import (CSA_BF16, CSA_F32, CSA_K_ATTN_DQ, CSA_K_ATTN_FWD, CSA_K_ATTN_REDUCE, CSA_K_ATTN_ROWS,
                   CSA_K_COMPRESS_BWD, CSA_K_COMPRESS_EPI, CSA_K_COMPRESS_FWD, CSA_K_INDEX_TOPK, CSA_K_LOSS_KEYS, CSA_K_LOSS_QUERY,
                   CSA_K_LOSS_REDUCE, EXPORTS, CSAError, csa_compress,
                   csa_compress_bwd, csa_compress_bwd_workspace, csa_dims,
                   csa_dsa_gqa_bwd, csa_dsa_gqa_fwd, csa_dsa_gqa_workspace, csa_gqa_dims, csa_index_topk, csa_index_topk_workspace, csa_indexer_loss,
                   csa_indexer_loss_dense, csa_indexer_loss_dense_workspace, csa_indexer_loss_workspace, csa_kernel_name,
                   csa_last_error, csa_sparse_attn_bwd, csa_sparse_attn_bwd_noalloc, csa_sparse_attn_fwd_strided, csa_sparse_attn_bwd_strided, csa_attn_strides, attn_strides_of,
                   csa_compress_strided, csa_compress_bwd_strided, csa_compress_strides, compress_strides_of,
                   csa_index_topk_strided, csa_index_strides, index_strides_of, csa_sparse_attn_bwd_query_block, csa_sparse_attn_bwd_workspace,
                   csa_sparse_attn_fwd,
                   csa_timing_enable, csa_timing_read, csa_version, dims_of, kprime, load, make_dims,
                   n_compressed, LIB_PATH)

__all__ = ["CSA_BF16", "CSA_F32", "CSA_K_ATTN_DQ", "CSA_K_ATTN_FWD", "CSA_K_ATTN_REDUCE", "CSA_K_ATTN_ROWS",
           "CSA_K_COMPRESS_BWD", "CSA_K_COMPRESS_EPI", "CSA_K_COMPRESS_FWD", "CSA_K_INDEX_TOPK", "CSA_K_LOSS_KEYS", "CSA_K_LOSS_QUERY",
           "CSA_K_LOSS_REDUCE", "EXPORTS", "CSAError", "csa_compress",
           "csa_compress_bwd", "csa_compress_bwd_workspace", "csa_dims",
           "csa_dsa_gqa_bwd", "csa_dsa_gqa_fwd", "csa_dsa_gqa_workspace", "csa_gqa_dims", "csa_index_topk", "csa_index_topk_workspace", "csa_indexer_loss",
           "csa_indexer_loss_dense", "csa_indexer_loss_dense_workspace", "csa_indexer_loss_workspace", "csa_kernel_name",
           "csa_last_error", "csa_sparse_attn_bwd", "csa_sparse_attn_bwd_noalloc", "csa_sparse_attn_fwd_strided", "csa_sparse_attn_bwd_strided", "csa_attn_strides", "attn_strides_of",
           "csa_compress_strided", "csa_compress_bwd_strided", "csa_compress_strides", "compress_strides_of",
           "csa_index_topk_strided", "csa_index_strides", "index_strides_of", "csa_sparse_attn_bwd_query_block", "csa_sparse_attn_bwd_workspace",
           "csa_sparse_attn_fwd",
           "csa_timing_enable", "csa_timing_read", "csa_version", "dims_of", "kprime", "load", "make_dims",
           "n_compressed", "LIB_PATH"]
