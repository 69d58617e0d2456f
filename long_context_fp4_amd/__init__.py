"""FP4 compressed global KV cache and sparse decode attention for AMD MI355X.

The compute path is the HIP library ``libcsa2fp4.so`` (gfx950 kernels behind a
C ABI, declared in ``include/csa2fp4.h``). This package holds its thin ctypes
binding (argument marshalling only; PyTorch supplies device memory and the
stream) and the seeded synthetic inputs used by the tests and the benchmark.
"""
from .binding import (  # noqa: F401
    CSA2_FULL, CSA2_REINDEX, CSA2_REUSE, CSA2_NOALLOC_SCRATCH_BYTES, CSA2_SCORE_DOT, CSA2_SCORE_RELU_W, CSA2_SCORE_QMX8,
    Csa2Error, Workspace, bytes_per_token, cache_append, cache_write, decode_layer, decode_layer_noalloc, indexer_topk,
    lib, library_path, prefill_layer, set_profile_events, sparse_attention, swa_attention, swa_write,
)
