"""MI355X-native (gfx950) forward hot path of MiniMax Sparse Attention (MSA).

The compute lives in the HIP/C-ABI library ``libmsa.so`` built from ``csrc/``
(``python -m block_sparse_gqa_02_amd.build``); ``binding`` marshals arguments
to it under the C names, ``configs`` describes the workloads and ``inputs``
draws seeded synthetic inputs.  The library is loaded on first use.
"""
from . import configs, inputs  # noqa: F401
from .binding import (Problem, MsaError, abi_version, decode_workspace,  # noqa: F401
                      msa_dense_attn_decode,
                      msa_dense_attn_prefill, msa_index_block_scores,
                      msa_index_block_scores_paged, msa_index_topk_fused,
                      msa_index_kl_backward, msa_index_topk_fused_paged,
                      msa_sparse_attn_decode,
                      msa_sparse_attn_prefill_backward,
                      msa_sparse_attn_decode_paged, msa_sparse_attn_prefill, msa_topk_blocks,
                      msa_sparse_attn_prefill_status_offset, msa_set_wait_limit,
                      msa_sparse_attn_decode_static,
                      msa_workspace_bytes)
