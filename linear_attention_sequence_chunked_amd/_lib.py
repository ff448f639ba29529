"""ctypes binding of libkda.so (declared in include/kda.h).  Marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP = 0, 1, 2, 3
KDA_DTYPE_BF16, KDA_DTYPE_F32 = 0, 1
EXPORTED = ("kda_chunk_prefill", "kda_chunk_prefill_checkpointed", "kda_decode_step",
            "kda_spec_verify", "kda_spec_commit", "kda_chunk_prefill_segmented",
            "kda_prefill_segmented_workspace", "kda_chunk_prefill_segmented_noalloc",
            "kda_noalloc_scratch_bytes", "kda_prefill_segment_plan", "kda_prefill_backward",
            "kda_prefill_backward_workspace", "kda_status_string", "kda_last_error",
            "kda_abi_version")


class KdaParams(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("log_alpha_floor", ctypes.c_float), ("scale", ctypes.c_float)]


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status
        self.detail = detail


_lib = None


def load() -> ctypes.CDLL:
    """Load libkda.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m linear_attention_sequence_chunked_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.kda_chunk_prefill.argtypes = [ctypes.POINTER(KdaParams), P, P, P, P, P, P, P,
                                      ctypes.POINTER(I32), I32, P, P, P, P]
    lib.kda_chunk_prefill.restype = ctypes.c_int
    lib.kda_chunk_prefill_checkpointed.argtypes = [ctypes.POINTER(KdaParams), P, P, P, P, P, P,
                                                   P, ctypes.POINTER(I32), I32, P, P, P, I32, P,
                                                   P]
    lib.kda_chunk_prefill_checkpointed.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [ctypes.POINTER(KdaParams), P, P, P, P, P, P, I32, P, P, P]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_spec_verify.argtypes = [ctypes.POINTER(KdaParams), P, P, P, P, P, P, I32, I32, P, P,
                                    P]
    lib.kda_spec_verify.restype = ctypes.c_int
    lib.kda_spec_commit.argtypes = [ctypes.POINTER(KdaParams), P, P, P, P, I32, I32, P, P, P]
    lib.kda_spec_commit.restype = ctypes.c_int
    lib.kda_chunk_prefill_segmented.argtypes = [ctypes.POINTER(KdaParams), P, P, P, P, P, P,
                                                ctypes.POINTER(I32), I32, P, P, P, I32, P,
                                                ctypes.c_int64, P]
    lib.kda_chunk_prefill_segmented.restype = ctypes.c_int
    lib.kda_prefill_segmented_workspace.argtypes = [ctypes.POINTER(KdaParams),
                                                    ctypes.POINTER(I32), I32, I32]
    lib.kda_prefill_segmented_workspace.restype = ctypes.c_int64
    lib.kda_chunk_prefill_segmented_noalloc.argtypes = [
        ctypes.POINTER(KdaParams), P, P, P, P, P, P, ctypes.POINTER(I32), I32, P, P, P, I32, P]
    lib.kda_chunk_prefill_segmented_noalloc.restype = ctypes.c_int
    lib.kda_noalloc_scratch_bytes.argtypes = []
    lib.kda_noalloc_scratch_bytes.restype = ctypes.c_int64
    lib.kda_prefill_segment_plan.argtypes = [ctypes.POINTER(KdaParams), ctypes.POINTER(I32), I32]
    lib.kda_prefill_segment_plan.restype = I32
    lib.kda_prefill_backward.argtypes = [ctypes.POINTER(KdaParams), P, P, P, P, P, P, P,
                                         ctypes.POINTER(I32), I32, P, P, P, P, P, P, P, P, P,
                                         P, P, ctypes.c_int64, P]
    lib.kda_prefill_backward.restype = ctypes.c_int
    lib.kda_prefill_backward_workspace.argtypes = [ctypes.POINTER(KdaParams),
                                                   ctypes.POINTER(I32), I32]
    lib.kda_prefill_backward_workspace.restype = ctypes.c_int64
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = I32
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != KDA_OK:
        lib = load()
        raise KdaError(status, lib.kda_last_error().decode() or
                       lib.kda_status_string(status).decode())


def params(dtype: int, H: int, dk: int, dv: int, floor: float = -0.3, scale: float = 1.0,
           chunk: int = 16) -> KdaParams:
    return KdaParams(dtype, H, dk, dv, chunk, floor, scale)
