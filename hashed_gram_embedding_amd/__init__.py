"""Hashed N-gram embedding layer (Engram-style) on AMD Instinct MI355X.

The layer runs in ``libngram.so`` (hand-written HIP kernels for gfx950,
C-ABI in ``include/ngram.h``); ``hashed_gram_embedding_amd.ngram`` is its
ctypes binding.  Importing this package loads the library and fails loudly
when it has not been built.
"""
from . import ngram  # noqa: F401
from .ngram import (ADD_RESIDUAL, BF16, F32, FP8_E4M3, KEEP_FOR_BACKWARD, MEM_ROWS,  # noqa: F401
                    MEM_TILES16, PREFETCHED, UPDATE_STATE, W_D_MEM, W_MEM_D, NgramConfig, NgramError,
                    make_config,
                    ngram_backward, ngram_backward_timed, ngram_backward_workspace_size,
                    ngram_causal_conv, ngram_compress_ids, ngram_config_validate, ngram_forward,
                    ngram_forward_noalloc, ngram_forward_prefetch, ngram_forward_timed,
                    ngram_forward_workspace_size,
                    ngram_forward_workspace_view, ngram_gate, ngram_gate_workspace_size,
                    ngram_gather, ngram_hash)

ngram.lib()
