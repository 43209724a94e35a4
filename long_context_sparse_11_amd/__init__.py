"""MI355X-native DeepSeek-V4 Compressed Sparse Attention (CSA) and Heavily
Compressed Attention (HCA).

The computation lives in the HIP library ``libcsa.so`` (C ABI in
include/csa.h); ``binding`` marshals torch tensors into it.  ``synth`` holds
the seeded synthetic workloads.
"""
from .binding import (  # noqa: F401
    CsaError,
    csa_attn_ws_bytes,
    csa_compress,
    csa_compress_batch,
    csa_compress_kvfp8,
    csa_dequantize_kv_fp8,
    csa_kv_fp8_row_bytes,
    csa_quantize_kv_fp8,
    csa_sparse_attn_kvfp8,
    hca_attn_kvfp8,
    csa_compress_ws_bytes,
    csa_decode_advance,
    csa_decode_index_scores,
    csa_decode_index_scores_mxfp4,
    csa_decode_index_topk,
    csa_decode_index_topk_noalloc,
    csa_window_row,
    csa_decode_index_topk_mxfp4,
    csa_index_scores_mxfp4,
    csa_index_topk_mxfp4,
    csa_quantize_mxfp4,
    csa_index_scores,
    csa_index_topk,
    csa_index_topk_ws_bytes,
    csa_output_proj,
    csa_sparse_attn,
    hca_attn,
    hca_decode_attn,
    hca_decode_attn_kvfp8,
    hca_decode_attn_ws_bytes,
    swa_decode_attn,
    swa_decode_attn_ws_bytes,
    lib,
)
