"""MI355X-native structured-sparse plus low-rank linear layer.

The compute lives in ``libsra.so`` (hand-written HIP for gfx950, C ABI in ``include/sra.h``);
this package only marshals torch tensors into those calls.  Importing it does not load the
library; the first call does, and raises if it has not been built.
"""
from .api import (SparseMatrix, bwd_workspace, ffa_bwd_workspace, ffa_fwd_workspace, compress, compress_ffi, compress_pair,  # noqa: F401
                  compress_pair_tiled, masked_weight_grad, nm_axpby, tile_bytes,
                  double_prune, ffi_tile, ffi_transpose, fwd_workspace, meta_words, nm_tile, sparse_lora_bwd,
                  sparse_lora_bwd_ffa, sparse_lora_fwd, sparse_lora_fwd_ffa, time_next_kernel,
                  set_tuning, reset_tuning, tuned)
