"""ctypes view of libnsa_sel.so (include/nsa_sel.h).  No computation here."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnsa_sel.so")

NSA_OK, NSA_ERR_INVALID_ARG, NSA_ERR_UNSUPPORTED, NSA_ERR_WORKSPACE, NSA_ERR_HIP = range(5)
NSA_F32, NSA_BF16 = 0, 1
NSA_DENSE, NSA_PACKED = 0, 1

# Every symbol include/nsa_sel.h declares.
EXPORTS = (
    "nsa_sel_fwd",
    "nsa_sel_bwd",
    "nsa_sel_bwd_noalloc",
    "nsa_sel_bwd_workspace_bytes",
    "nsa_sel_bwd_prepare",
    "nsa_sel_bwd_prepare_lists",
    "nsa_sel_bwd_prepare_delta",
    "nsa_sel_bwd_dq",
    "nsa_sel_bwd_dkdv",
    "nsa_sel_bwd_dkdv_blocks",
    "nsa_sel_bwd_dkdv_reduce",
    "nsa_sel_delta",
    "nsa_sel_invert",
    "nsa_sel_invert_tokens_capacity",
    "nsa_sel_check_block_idx",
    "nsa_sel_fwd_sink",
    "nsa_sel_bwd_dsink",
    "nsa_sel_wait_timeouts",
    "nsa_sel_bwd_ds_handoff",
    "nsa_build_git",
    "nsa_status_string",
    "nsa_last_error",
)


class Problem(ctypes.Structure):
    """Mirror of struct nsa_sel_problem."""
    _fields_ = [
        ("layout", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("S", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("n_seqs", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("window", ctypes.c_int32),
        ("strided", ctypes.c_int32),
        ("stride_q", ctypes.c_int64 * 3),
        ("stride_k", ctypes.c_int64 * 3),
        ("stride_v", ctypes.c_int64 * 3),
        ("stride_o", ctypes.c_int64 * 3),
        ("stride_do", ctypes.c_int64 * 3),
        ("stride_dq", ctypes.c_int64 * 3),
        ("stride_dk", ctypes.c_int64 * 3),
        ("stride_dv", ctypes.c_int64 * 3),
        ("Tk", ctypes.c_int32),
        ("sched_policy", ctypes.c_int32),
    ]


class NsaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: {status_string(status)} ({status}): {detail}")
        self.status = status


_lib = None


def load():
    """Load the library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_attention_nsa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, ip, fp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    st, sz = ctypes.c_int, ctypes.c_size_t
    lib.nsa_sel_fwd.argtypes = [P, vp, vp, vp, ip, ip, vp, fp, vp]
    lib.nsa_sel_fwd.restype = st
    lib.nsa_sel_bwd.argtypes = [P, vp, vp, vp, vp, fp, vp, ip, ip, vp, vp, vp, vp, sz, vp]
    lib.nsa_sel_bwd.restype = st
    lib.nsa_sel_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, fp, vp, ip, ip, vp, vp, vp, vp]
    lib.nsa_sel_bwd_noalloc.restype = st
    lib.nsa_sel_bwd_workspace_bytes.argtypes = [P]
    lib.nsa_sel_bwd_workspace_bytes.restype = sz
    lib.nsa_sel_bwd_prepare.argtypes = [P, vp, vp, ip, ip, vp, sz, vp]
    lib.nsa_sel_bwd_prepare.restype = st
    lib.nsa_sel_bwd_prepare_lists.argtypes = [P, ip, ip, vp, sz, vp]
    lib.nsa_sel_bwd_prepare_lists.restype = st
    lib.nsa_sel_bwd_prepare_delta.argtypes = [P, vp, vp, ip, vp, sz, vp]
    lib.nsa_sel_bwd_prepare_delta.restype = st
    lib.nsa_sel_bwd_dq.argtypes = [P, vp, vp, vp, vp, fp, ip, ip, vp, vp, sz, vp]
    lib.nsa_sel_bwd_dq.restype = st
    lib.nsa_sel_bwd_dkdv.argtypes = [P, vp, vp, vp, vp, fp, ip, vp, vp, vp, sz, vp]
    lib.nsa_sel_bwd_dkdv.restype = st
    lib.nsa_sel_bwd_dkdv_blocks.argtypes = [P, vp, vp, vp, vp, fp, ip, vp, vp, vp, sz, vp]
    lib.nsa_sel_bwd_dkdv_blocks.restype = st
    lib.nsa_sel_bwd_dkdv_reduce.argtypes = [P, ip, vp, vp, vp, sz, vp]
    lib.nsa_sel_bwd_dkdv_reduce.restype = st
    lib.nsa_sel_delta.argtypes = [P, vp, vp, ip, fp, vp]
    lib.nsa_sel_delta.restype = st
    lib.nsa_sel_invert.argtypes = [P, ip, ip, ip, ip, vp, sz, vp]
    lib.nsa_sel_invert.restype = st
    lib.nsa_sel_invert_tokens_capacity.argtypes = [P]
    lib.nsa_sel_invert_tokens_capacity.restype = sz
    lib.nsa_sel_check_block_idx.argtypes = [P, ip, ip, vp, vp]
    lib.nsa_sel_check_block_idx.restype = st
    lib.nsa_sel_fwd_sink.argtypes = [P, vp, vp, vp, ip, ip, fp, vp, fp, vp]
    lib.nsa_sel_fwd_sink.restype = st
    lib.nsa_sel_bwd_dsink.argtypes = [P, fp, fp, ip, fp, vp, sz, vp]
    lib.nsa_sel_bwd_dsink.restype = st
    lib.nsa_sel_wait_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.nsa_sel_wait_timeouts.restype = st
    lib.nsa_sel_bwd_ds_handoff.argtypes = [P]
    lib.nsa_sel_bwd_ds_handoff.restype = ctypes.c_int32
    lib.nsa_build_git.argtypes = []
    lib.nsa_build_git.restype = ctypes.c_char_p
    lib.nsa_status_string.argtypes = [ctypes.c_int]
    lib.nsa_status_string.restype = ctypes.c_char_p
    lib.nsa_last_error.argtypes = []
    lib.nsa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().nsa_status_string(status).decode()


def last_error() -> str:
    return load().nsa_last_error().decode()


def check(fn: str, status: int) -> None:
    if status != NSA_OK:
        raise NsaError(fn, status, last_error())
