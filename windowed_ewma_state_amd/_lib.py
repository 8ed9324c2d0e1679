"""ctypes view of libsfa.so (the C ABI in include/sfa.h).

Loading fails loudly when the library has not been built: there is no CPU
fallback behind these entry points.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsfa.so")

SFA_OK, SFA_ERR_INVALID_ARG, SFA_ERR_UNSUPPORTED, SFA_ERR_HIP, SFA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
SFA_NOALLOC_SCRATCH_BYTES = 16 << 20
SFA_F32, SFA_BF16 = 0, 1
SFA_PREFILL_SCAN, SFA_PREFILL_ATTEND, SFA_PREFILL_SINGLE_PASS = 1, 2, 4

# every symbol include/sfa.h declares
EXPORTS = ("sfa_status_string", "sfa_abi_version", "sfa_prefill_workspace_size", "sfa_prefill",
           "sfa_prefill_part", "sfa_prefill_qh", "sfa_prefill_rm", "sfa_prefill_noalloc",
           "sfa_decode_step", "sfa_decode_step_qh", "sfa_decode_step_rm", "sfa_enhance_workspace_size",
           "sfa_enhance", "sfa_enhance_pool_bytes", "sfa_enhance_prepare_pool", "sfa_enhance_prepared",
           "sfa_decode_step_enhance")

_lib = None


class SFAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m windowed_ewma_state_amd.build` "
                "(hipcc, gfx950). The SFA ops have no CPU fallback.")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.sfa_status_string.argtypes = [I]
        L.sfa_status_string.restype = ctypes.c_char_p
        L.sfa_abi_version.argtypes = []
        L.sfa_abi_version.restype = I
        L.sfa_prefill_workspace_size.argtypes = [I, I, I, I]
        L.sfa_prefill_workspace_size.restype = Z
        L.sfa_prefill.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P, Z, P]
        L.sfa_prefill.restype = I
        L.sfa_prefill_part.argtypes = [I, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I,
                                       P, Z, P]
        L.sfa_prefill_part.restype = I
        L.sfa_prefill_qh.argtypes = L.sfa_prefill.argtypes
        L.sfa_prefill_qh.restype = I
        L.sfa_prefill_rm.argtypes = L.sfa_prefill.argtypes
        L.sfa_prefill_rm.restype = I
        L.sfa_prefill_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P]
        L.sfa_prefill_noalloc.restype = I
        L.sfa_decode_step.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P]
        L.sfa_decode_step.restype = I
        L.sfa_decode_step_qh.argtypes = L.sfa_decode_step.argtypes
        L.sfa_decode_step_qh.restype = I
        L.sfa_decode_step_rm.argtypes = L.sfa_decode_step.argtypes
        L.sfa_decode_step_rm.restype = I
        L.sfa_enhance_workspace_size.argtypes = [I, I, I]
        L.sfa_enhance_workspace_size.restype = Z
        L.sfa_enhance.argtypes = [P, P, P, P, P, ctypes.c_longlong, P, I, I, I, I, I, I,
                                  F, F, F, F, F, I, I, I, I, P, Z, P]
        L.sfa_enhance.restype = I
        L.sfa_enhance_pool_bytes.argtypes = [I, I]
        L.sfa_enhance_pool_bytes.restype = Z
        L.sfa_enhance_prepare_pool.argtypes = [P, ctypes.c_longlong, I, I, I, P, Z, P]
        L.sfa_enhance_prepare_pool.restype = I
        L.sfa_enhance_prepared.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, I,
                                           F, F, F, F, F, I, I, I, I, P, Z, P]
        L.sfa_enhance_prepared.restype = I
        L.sfa_decode_step_enhance.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, I, P,
                                              I, I, I, I, I, I, F, I, I, F, F, F, F, F, I, I, I, I, P]
        L.sfa_decode_step_enhance.restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sfa_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != SFA_OK:
        raise SFAError(status, where)
