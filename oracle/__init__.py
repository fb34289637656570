"""CPU oracle for CSA / HCA (test infrastructure only).

Only the test suite, the repository entry module's smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links it.
"""

from .csa_oracle import *  # noqa: F401,F403
from .csa_oracle import (  # noqa: F401  (explicit re-exports for linters)
    visible_entries, LayerReads, layer_reads, compress_overlap, compress_pool,
    compress_weights_overlap, compress_weights_pool, index_scores, topk_select,
    index_topk, attend_entries, csa_attend, hca_attend, hca_layer, csa_layer,
    CsaDecodeState, HcaDecodeState, block_geometry, default_scale, window_rows, rms_norm, rope_frequencies,
    rope, norm_rope, csa_attend_rope, grouped_out_proj, attend_entries_backward, csa_attend_backward,
    hca_attend_backward, compress_overlap_backward, compress_pool_backward, fp8_e4m3_encode, kv_fp8_encode,
    kv_fp8_decode,
)
