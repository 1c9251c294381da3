"""ctypes declarations of libsra's C ABI (include/sra.h).  Marshalling only."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsra.so")

SRA_OK, SRA_ERR_INVALID_ARG, SRA_ERR_UNSUPPORTED, SRA_ERR_WORKSPACE, SRA_ERR_HIP = 0, -1, -2, -3, -4
STATUS_NAMES = {0: "SRA_OK", -1: "SRA_ERR_INVALID_ARG", -2: "SRA_ERR_UNSUPPORTED",
                -3: "SRA_ERR_WORKSPACE", -4: "SRA_ERR_HIP"}
SRA_BF16, SRA_F32 = 0, 1
SRA_FMT_NM, SRA_FMT_ELL, SRA_FMT_CSR, SRA_FMT_NM_TILED, SRA_FMT_FFI_TILED = 0, 1, 2, 3, 4
SRA_GRAD_DX, SRA_GRAD_DA, SRA_GRAD_DB, SRA_DX_NO_ADAPTER = 1, 2, 4, 8
SRA_NOALLOC_SCRATCH_BYTES = 64 << 20
SRA_TUNE_KEYS = {"spmm_config": 1, "spmm_splits": 2, "spmm_fuse": 3, "engine": 4, "decode_rows": 5,
                 "rows_slices": 6, "grads_slices": 7}
SRA_ENGINE_SMFMAC, SRA_ENGINE_DENSE_MFMA = 0, 1

# every symbol include/sra.h declares
EXPORTS = (
    "sra_abi_version", "sra_last_error", "sra_nm_meta_words", "sra_compress", "sra_double_prune",
    "sra_compress_pair", "sra_compress_pair_tiled", "sra_nm_tile_bytes", "sra_nm_tile",
    "sra_masked_weight_grad", "sra_nm_axpby",
    "sra_compress_ffi", "sra_ffi_transpose_workspace", "sra_ffi_transpose", "sra_ffi_tile_size",
    "sra_ffi_tile", "sra_fwd_workspace",
    "sra_sparse_lora_fwd", "sra_bwd_workspace", "sra_sparse_lora_bwd", "sra_sparse_lora_bwd_noalloc",
    "sra_ffa_fwd_workspace", "sra_sparse_lora_fwd_ffa", "sra_ffa_bwd_workspace", "sra_sparse_lora_bwd_ffa",
    "sra_time_next_kernel", "sra_set_tuning",
)
SRA_KERNEL_COMPRESS, SRA_KERNEL_DOUBLE_PRUNE, SRA_KERNEL_SPMM24 = 1, 2, 3
SRA_KERNEL_ADAPTER, SRA_KERNEL_DECODE24, SRA_KERNEL_SPMM_FFI = 4, 5, 6
SRA_KERNEL_FFI_DENSIFY, SRA_KERNEL_WEIGHT_GRAD, SRA_KERNEL_NM_UPDATE = 7, 8, 9


class SraSparse(ctypes.Structure):
    _fields_ = [
        ("format", c_int32), ("dtype", c_int32), ("rows", c_int64), ("cols", c_int64),
        ("n", c_int32), ("m", c_int32), ("k", c_int32), ("nnz", c_int64),
        ("values", c_void_p), ("meta", c_void_p), ("index", c_void_p), ("row_ptr", c_void_p),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load libsra.so (after torch, so both share torch's HIP runtime).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- loads the HIP runtime the library must share

    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m sparse_rank_adapter_amd.build`")
    lib = ctypes.CDLL(path)
    P = POINTER(SraSparse)
    sig = {
        "sra_abi_version": (c_int32, []),
        "sra_last_error": (c_char_p, []),
        "sra_nm_meta_words": (c_int64, [c_int64, c_int32, c_int32]),
        "sra_compress": (c_int32, [c_void_p, c_int32, c_int64, c_int64, c_int32, c_int32, P, c_void_p]),
        "sra_double_prune": (c_int32, [P, P, c_void_p]),
        "sra_compress_pair": (c_int32, [c_void_p, c_int32, c_int64, c_int64, c_int32, c_int32, P, P, c_void_p]),
        "sra_compress_pair_tiled": (c_int32, [c_void_p, c_int32, c_int64, c_int64, c_int32, c_int32, P, P, c_void_p]),
        "sra_nm_axpby": (c_int32, [c_void_p, c_float, c_void_p, c_float, c_void_p, c_int64, c_int32, c_void_p]),
        "sra_masked_weight_grad": (c_int32, [P, c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
        "sra_nm_tile_bytes": (c_int32, [c_int64, c_int64, c_int32, c_int32, POINTER(c_size_t), POINTER(c_size_t)]),
        "sra_nm_tile": (c_int32, [P, P, c_void_p]),
        "sra_compress_ffi": (c_int32, [c_void_p, c_int32, c_int64, c_int64, c_int32, P, c_void_p]),
        "sra_ffi_transpose_workspace": (c_int32, [c_int64, c_int64, c_int32, POINTER(c_size_t)]),
        "sra_ffi_transpose": (c_int32, [P, P, c_void_p, c_size_t, c_void_p]),
        "sra_ffi_tile_size": (c_int32, [c_int64, c_int64, c_int64, POINTER(c_size_t), POINTER(c_size_t)]),
        "sra_ffi_tile": (c_int32, [P, P, c_void_p]),
        "sra_fwd_workspace": (c_int32, [P, c_int64, c_int32, POINTER(c_size_t)]),
        "sra_sparse_lora_fwd": (c_int32, [P, c_void_p, c_int64, c_void_p, c_void_p, c_int32, c_void_p,
                                          c_void_p, c_void_p, c_size_t, c_void_p]),
        "sra_bwd_workspace": (c_int32, [P, c_int64, c_int32, c_uint32, POINTER(c_size_t)]),
        "sra_sparse_lora_bwd": (c_int32, [P, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
                                          c_int32, c_uint32, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_size_t, c_void_p]),
        "sra_sparse_lora_bwd_noalloc": (c_int32, [P, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                                  c_void_p, c_int32, c_uint32, c_void_p, c_void_p,
                                                  c_void_p, c_void_p, c_void_p]),
        "sra_ffa_fwd_workspace": (c_int32, [P, c_int64, P, POINTER(c_size_t)]),
        "sra_sparse_lora_fwd_ffa": (c_int32, [P, c_void_p, c_int64, P, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_size_t, c_void_p]),
        "sra_ffa_bwd_workspace": (c_int32, [P, c_int64, P, c_uint32, POINTER(c_size_t)]),
        "sra_sparse_lora_bwd_ffa": (c_int32, [P, c_void_p, c_void_p, c_int64, c_void_p, P, c_void_p,
                                              c_uint32, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_size_t, c_void_p]),
        "sra_time_next_kernel": (c_int32, [c_int32, c_void_p, c_void_p]),
        "sra_set_tuning": (c_int32, [c_int32, c_int32]),
    }
    assert set(sig) == set(EXPORTS)
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class SraError(RuntimeError):
    def __init__(self, call: str, status: int, msg: str):
        super().__init__(f"{call} -> {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(call: str, status: int):
    if status != SRA_OK:
        raise SraError(call, status, load().sra_last_error().decode())
