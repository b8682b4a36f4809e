"""ctypes loader of the HIP library ``libssm_scan.so`` (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssm_scan.so")

SSM_F32 = 0
SSM_BF16 = 1

# every symbol include/ssm_scan.h declares
EXPORTS = ("ssm_abi_version", "ssm_status_string", "ssm_last_error", "ssm_scan_chunk_len",
           "ssm_scan_chunk_states_bytes", "ssm_scan_fwd_workspace_bytes", "ssm_scan_fwd",
           "ssm_scan_fwd_ex", "ssm_scan_bwd_workspace_bytes", "ssm_scan_bwd", "ssm_scan_bwd_ex",
           "ssm_state_update", "ssm_state_update_ex", "ssm_scan_fwd_conv",
           "ssm_scan_bwd_conv_workspace_bytes", "ssm_scan_bwd_conv", "ssm_scan_fwd_plan",
           "ssm_scan_fwd_noalloc", "ssm_affine_scan")


class FwdPlan(ctypes.Structure):
    """ssm_fwd_plan: kernel (0 all-purpose, 1 wave-specialised), channels per
    workgroup, sequence segments and their length."""
    _fields_ = [("kernel", ctypes.c_int32), ("tile_channels", ctypes.c_int32),
                ("segments", ctypes.c_int64), ("segment_len", ctypes.c_int64),
                ("first_pass_len", ctypes.c_int64)]

# option bits of the *_ex entry points
FLAG_ZOH = 1
FLAG_REVERSE = 2
FLAG_DELTA_PER_TOKEN = 4
FLAG_ACCUMULATE = 8

_lib = None


class SSMError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the built library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                          "(run selective_state_space_10_amd/build.py or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    I64, INT, P = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.ssm_abi_version.restype = INT
    lib.ssm_abi_version.argtypes = []
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_status_string.argtypes = [INT]
    lib.ssm_last_error.restype = ctypes.c_char_p
    lib.ssm_last_error.argtypes = []
    lib.ssm_scan_chunk_len.restype = I64
    lib.ssm_scan_chunk_len.argtypes = []
    lib.ssm_scan_chunk_states_bytes.restype = I64
    lib.ssm_scan_chunk_states_bytes.argtypes = [I64] * 4
    lib.ssm_scan_fwd_workspace_bytes.restype = I64
    lib.ssm_scan_fwd_workspace_bytes.argtypes = [I64] * 4 + [INT]
    lib.ssm_scan_bwd_workspace_bytes.restype = I64
    lib.ssm_scan_bwd_workspace_bytes.argtypes = [I64] * 4 + [INT]
    lib.ssm_scan_fwd.restype = INT
    lib.ssm_scan_fwd.argtypes = [I64] * 4 + [INT] + [P] * 8 + [INT] + [P] * 5 + [I64, P]
    lib.ssm_scan_bwd.restype = INT
    lib.ssm_scan_bwd.argtypes = [I64] * 4 + [INT] + [P] * 8 + [INT] + [P] * 14 + [I64, P]
    lib.ssm_state_update.restype = INT
    lib.ssm_state_update.argtypes = [I64] * 3 + [INT] + [P] * 9 + [INT, P, P]
    for name in ("ssm_scan_fwd", "ssm_scan_bwd", "ssm_state_update"):
        ex = getattr(lib, name + "_ex")
        ex.restype = INT
        ex.argtypes = getattr(lib, name).argtypes + [INT]
    lib.ssm_scan_fwd_conv.restype = INT
    lib.ssm_scan_fwd_conv.argtypes = [I64] * 4 + [INT] + [P] * 3 + [INT] + [P] * 7 + [INT] \
        + [P] * 5 + [I64, P, INT]
    lib.ssm_scan_bwd_conv_workspace_bytes.restype = I64
    lib.ssm_scan_bwd_conv_workspace_bytes.argtypes = [I64] * 4 + [INT]
    lib.ssm_scan_bwd_conv.restype = INT
    # h0, chunk_states, dy, dh_final, dx, dconv_w, dconv_b, ddelta, dA, dB, dC, dD, dz,
    # ddelta_bias, dh0, workspace
    lib.ssm_scan_bwd_conv.argtypes = [I64] * 4 + [INT] + [P] * 3 + [INT] + [P] * 7 + [INT] \
        + [P] * 16 + [I64, P, INT]
    lib.ssm_affine_scan.restype = INT
    lib.ssm_affine_scan.argtypes = [I64, I64, P, P, P, P, INT, P]
    lib.ssm_scan_fwd_noalloc.restype = INT
    lib.ssm_scan_fwd_noalloc.argtypes = [I64] * 4 + [INT] + [P] * 8 + [INT] + [P] * 5 + [INT]
    lib.ssm_scan_fwd_plan.restype = INT
    lib.ssm_scan_fwd_plan.argtypes = [I64] * 4 + [INT, INT, INT, ctypes.POINTER(FwdPlan)]
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        lib = load()
        msg = lib.ssm_last_error().decode() or lib.ssm_status_string(status).decode()
        raise SSMError(status, msg)
