"""MI355X (gfx950) compressed sparse attention: one CSA / HCA layer.

The compute lives in libcsa.so (hand-written HIP kernels behind the C ABI of
include/csa.h).  This package is its thin Python binding; torch provides
device memory and streams only.
"""

from ._binding import (  # noqa: F401
    CSA_BF16, CSA_F32, CsaError, LIB_PATH, csa_attend, csa_compress, csa_grouped_out_proj, csa_index_topk,
    csa_index_topk_mxfp4, csa_index_topk_noalloc, csa_norm_rope, csa_quantize_mxfp4, hca_attend, hca_layer,
    load_library, strerror, version, BlockPool, PagedCache, csa_paged_append, csa_paged_index_topk,
    csa_paged_attend, hca_paged_attend, csa_attend_backward, hca_attend_backward, csa_compress_backward,
    csa_quantize_kv_fp8, csa_attend_fp8kv, csa_attend_norm_rope,
    hca_attend_norm_rope,
)

__all__ = [
    "csa_compress", "csa_index_topk", "csa_index_topk_noalloc", "csa_index_topk_mxfp4", "csa_quantize_mxfp4",
    "csa_norm_rope", "csa_grouped_out_proj", "csa_attend", "hca_attend", "hca_layer",
    "load_library", "version", "strerror", "CsaError", "CSA_F32", "CSA_BF16", "LIB_PATH",
    "BlockPool", "PagedCache", "csa_paged_append", "csa_paged_index_topk", "csa_paged_attend", "hca_paged_attend",
    "csa_attend_backward", "hca_attend_backward", "csa_compress_backward", "csa_quantize_kv_fp8", "csa_attend_fp8kv",
    "csa_attend_norm_rope", "hca_attend_norm_rope",
]
