"""ctypes view of include/ra.h.  Loading fails loudly if libra.so is missing:
there is no fallback implementation of any entry point."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libra.so")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP, RA_ERR_WORKSPACE = range(5)
LAYOUT_IDS = {"contiguous": 0, "zigzag": 1, "stripe": 2, "zigzag_varlen": 3, "stripe_varlen": 4}
DTYPE_F32, DTYPE_BF16 = 0, 1


class ra_seg(C.Structure):
    _fields_ = [("begin", C.c_int64), ("stride", C.c_int64), ("len", C.c_int64)]


class ra_posmap(C.Structure):
    _fields_ = [("nseg", C.c_int32), ("seg", ra_seg * 2)]


class ra_tensor(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("stride_b", C.c_int64), ("stride_t", C.c_int64), ("stride_h", C.c_int64)]


class ra_problem(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
        ("dtype", C.c_int32), ("softmax_scale", C.c_float), ("causal", C.c_int32),
        ("cu_seqlens", C.c_void_p), ("cu_seqlens_host", C.c_void_p),
        ("num_seqs", C.c_int32), ("seq_len", C.c_int64),
    ]


class ra_launch_time(C.Structure):
    _fields_ = [("kernel_id", C.c_int32), ("step", C.c_int32), ("ms", C.c_float)]


P = C.POINTER
_SIGS = {
    "ra_block_attn_fwd": [P(ra_problem), ra_tensor, C.c_int64, ra_posmap, ra_tensor, ra_tensor, C.c_int64,
                          ra_posmap, ra_tensor, C.c_void_p, C.c_void_p],
    "ra_lse_merge": [P(ra_problem), C.c_int64, ra_tensor, C.c_void_p, ra_tensor, C.c_void_p, C.c_void_p],
    "ra_bwd_preprocess": [P(ra_problem), C.c_int64, ra_tensor, ra_tensor, C.c_void_p, C.c_void_p],
    "ra_block_attn_bwd": [P(ra_problem), ra_tensor, C.c_int64, ra_posmap, ra_tensor, ra_tensor, C.c_int64,
                          ra_posmap, ra_tensor, C.c_void_p, C.c_void_p, ra_tensor, ra_tensor, ra_tensor,
                          C.c_void_p],
    "ra_ring_fwd": [P(ra_problem), C.c_int32, C.c_int32, C.c_int32, ra_tensor, ra_tensor, ra_tensor, C.c_int64,
                    ra_tensor, C.c_void_p, ra_tensor, C.c_void_p],
    "ra_ring_bwd": [P(ra_problem), C.c_int32, C.c_int32, C.c_int32, ra_tensor, ra_tensor, ra_tensor, C.c_int64,
                    ra_tensor, C.c_void_p, ra_tensor, ra_tensor, ra_tensor, ra_tensor, C.c_int64,
                    C.c_void_p, C.c_size_t, C.c_void_p],
    "ra_ring_bwd_noalloc": [P(ra_problem), C.c_int32, C.c_int32, C.c_int32, ra_tensor, ra_tensor, ra_tensor,
                            C.c_int64, ra_tensor, C.c_void_p, ra_tensor, ra_tensor, ra_tensor, ra_tensor, C.c_int64,
                            C.c_void_p],
    "ra_gathered_fwd": [P(ra_problem), C.c_int32, C.c_int32, C.c_int32, ra_tensor, ra_tensor, ra_tensor,
                        ra_tensor, C.c_void_p, ra_tensor, C.c_void_p],
    "ra_gathered_bwd": [P(ra_problem), C.c_int32, C.c_int32, C.c_int32, ra_tensor, ra_tensor, ra_tensor,
                        ra_tensor, C.c_void_p, ra_tensor, ra_tensor, ra_tensor, ra_tensor,
                        C.c_void_p, C.c_size_t, C.c_void_p],
    "ra_layout_positions": [C.c_int32, C.c_int64, C.c_int32, C.c_int32, P(C.c_int64)],
    "ra_layout_posmap": [C.c_int32, C.c_int64, C.c_int32, C.c_int32, P(ra_posmap)],
    "ra_layout_positions_cu": [C.c_int32, P(C.c_int32), C.c_int32, C.c_int32, C.c_int32, P(C.c_int64)],
    "ra_cast_f32_to_bf16": [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p],
    "ra_timing_begin": [C.c_int32],
    "ra_timing_end": [P(ra_launch_time), C.c_int32, P(C.c_int32)],
}

_lib = None


def lib():
    """The loaded libra.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python exact_long_context_ra_amd/build.py` (no CPU fallback exists)")
        L = C.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = C.c_int
        for name in ("ra_ring_workspace_bytes", "ra_ring_workspace_min_bytes"):
            getattr(L, name).argtypes = [P(ra_problem), C.c_int32, C.c_int32]
            getattr(L, name).restype = C.c_size_t
        for name in ("ra_gathered_workspace_bytes", "ra_gathered_workspace_min_bytes"):
            getattr(L, name).argtypes = [P(ra_problem), C.c_int32, C.c_int32, C.c_int32]
            getattr(L, name).restype = C.c_size_t
        L.ra_noalloc_scratch_bytes.argtypes = []
        L.ra_noalloc_scratch_bytes.restype = C.c_size_t
        for name in ("ra_status_str", "ra_kernel_name"):
            getattr(L, name).restype = C.c_char_p
        L.ra_status_str.argtypes = [C.c_int]
        L.ra_kernel_name.argtypes = [C.c_int32]
        L.ra_last_error.argtypes = []
        L.ra_last_error.restype = C.c_char_p
        L.ra_abi_version.argtypes = []
        L.ra_abi_version.restype = C.c_int
        _lib = L
    return _lib


class RAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{lib().ra_status_str(status).decode()}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != RA_OK:
        raise RAError(status, lib().ra_last_error().decode(errors="replace"))
