"""DeepSeek Sparse Attention prefill on one context-parallel rank, for AMD MI355X (gfx950).

The compute lives in libdsa.so (hand-written HIP kernels behind the C ABI of include/dsa.h);
this package only marshals torch tensors (device memory) and the current HIP stream into it.
"""
from .binding import (  # noqa: F401
    DSA_F32, DSA_BF16, DSA_FP8_E4M3, IN_SEQ, ROUND_ROBIN, DsaError, lib, library_path, library,
    checked_library_path,
    cp_sizes, build_cp_metadata, indexer_topk, indexer_topk_noalloc, indexer_topk_timed, indexer_topk_workspace,
    indexer_scores, topk_from_scores, sparse_attn, rerange, version, clock_probe, probe_mhz, lds_mfma_probe,
    lds_mfma_busy,
)
