"""MiniMax Sparse Attention (MSA) decode on AMD Instinct MI355X (gfx950).

A thin Python face over the C ABI of libmsa (include/msa.h): the functions
carry the ABI's names and take torch device tensors; all work runs in the
library's HIP kernels.
"""
from ._binding import (DTYPES, EXPORTS, MSA_ERR_BAD_DATA, MSA_ERR_HIP,  # noqa: F401
                       MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE,
                       MSA_FLAG_DEBUG_CHECKS, MSA_NOALLOC_SCRATCH_BYTES, MSA_OK, MSAError,
                       Pools, Problem, Tensors, describe, lib, library_path,
                       msa_build_page_table, msa_decode, msa_decode_noalloc, msa_index_score,
                       msa_insert_kv, msa_last_check_failure, msa_last_dispatch,
                       msa_last_hip_error, msa_select_blocks, msa_selftest_decoders,
                       msa_sparse_decode, msa_status_string, msa_workspace_bytes, pools,
                       problem, tensors)
