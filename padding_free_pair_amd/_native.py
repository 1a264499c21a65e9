"""ctypes declarations for libntpair.so (the C ABI of include/nt_pair.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libntpair.so")

NT_OK, NT_ERR_NULL, NT_ERR_INVALID, NT_ERR_OVERFLOW, NT_ERR_ALIGN, NT_ERR_WORKSPACE, \
    NT_ERR_DTYPE, NT_ERR_HIP = range(8)
STATUS_NAMES = {0: "NT_OK", 1: "NT_ERR_NULL", 2: "NT_ERR_INVALID", 3: "NT_ERR_OVERFLOW",
                4: "NT_ERR_ALIGN", 5: "NT_ERR_WORKSPACE", 6: "NT_ERR_DTYPE", 7: "NT_ERR_HIP"}
NT_F32, NT_BF16 = 0, 1
NT_TRANSITION_RELU_MLP, NT_TRANSITION_LN_SWIGLU = 0, 1

# Every symbol the header declares, for the export check.
EXPORTS = ("nt_partition_sizes", "nt_make_partition", "nt_partition_sizes_rect",
           "nt_make_partition_rect", "nt_decode_cells", "nt_pair_broadcast",
           "nt_pair_transition", "nt_pair_broadcast_transition", "nt_pair_transition_swiglu",
           "nt_pair_reduce",
           "nt_block_workspace_bytes", "nt_pair_block", "nt_pair_block_noalloc",
           "nt_pair_block_rect",
           "nt_chain_workspace_bytes", "nt_pair_chain", "nt_pair_block_ex", "nt_pair_chain_ex",
           "nt_block_backward_ex_workspace_bytes", "nt_pair_block_backward_ex",
           "nt_loss_workspace_bytes", "nt_pair_loss_eq5", "nt_pair_reduce_backward",
           "nt_pair_broadcast_backward", "nt_transition_backward_workspace_bytes",
           "nt_pair_transition_backward", "nt_block_backward_workspace_bytes",
           "nt_pair_block_backward", "nt_block_nl_workspace_bytes", "nt_pair_block_nl",
           "nt_block_backward_nl_workspace_bytes", "nt_pair_block_backward_nl", "nt_last_error",
           "nt_version")


class NtPartition(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32), ("B", ctypes.c_int32), ("n_max", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("T", ctypes.c_int64), ("cells", ctypes.c_int64),
        ("n_items", ctypes.c_int64),
        ("lengths", ctypes.c_void_p), ("single_offsets", ctypes.c_void_p),
        ("pair_offsets", ctypes.c_void_p), ("row_splits", ctypes.c_void_p),
        ("row_sample", ctypes.c_void_p), ("item_offsets", ctypes.c_void_p),
        ("tile_sample", ctypes.c_void_p), ("T_cols", ctypes.c_int64),
        ("col_lengths", ctypes.c_void_p), ("col_offsets", ctypes.c_void_p),
    ]


class NtBlockWeights(ctypes.Structure):
    _fields_ = [("Wa", ctypes.c_void_p), ("Wb", ctypes.c_void_p), ("W1", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("Wo", ctypes.c_void_p)]


class NtBlockGrads(ctypes.Structure):
    _fields_ = [("Wa", ctypes.c_void_p), ("Wb", ctypes.c_void_p), ("W1", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("Wo", ctypes.c_void_p)]


# nt_block_params / nt_block_param_grads: field names as in the header
PARAM_NAMES = ("Wa", "Wb", "Wo", "W1", "W2", "ln_gamma", "ln_beta", "W_gate", "W_up", "W_down")


class NtBlockParams(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("ln_eps", ctypes.c_float)] + \
        [(k, ctypes.c_void_p) for k in PARAM_NAMES]


class NtBlockParamGrads(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in PARAM_NAMES]


_lib = None


class NativeLibraryMissing(ImportError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NativeLibraryMissing(
            f"{LIB_PATH} is missing; build it with `python -m padding_free_pair_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    i32, i64, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    part = P(NtPartition)
    sig = {
        "nt_partition_sizes": [P(i32), i32, P(i64), P(i64), P(i32), P(sz)],
        "nt_make_partition": [P(i32), i32, vp, sz, vp, part],
        "nt_partition_sizes_rect": [P(i32), P(i32), i32, P(i64), P(i64), P(i64), P(sz)],
        "nt_make_partition_rect": [P(i32), P(i32), i32, vp, sz, vp, part],
        "nt_decode_cells": [part, vp, vp, vp, vp],
        "nt_pair_broadcast": [part, vp, vp, vp, i32, ctypes.c_int, vp],
        "nt_pair_transition": [part, vp, vp, vp, vp, i32, i32, ctypes.c_int, vp],
        "nt_pair_broadcast_transition": [part, vp, vp, vp, vp, vp, i32, i32, ctypes.c_int, vp],
        "nt_pair_transition_swiglu": [part, vp, vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_float,
                                      ctypes.c_int, vp],
        "nt_pair_reduce": [part, vp, vp, i32, ctypes.c_int, vp],
        "nt_block_workspace_bytes": [part, i32, i32, i32, ctypes.c_int, P(sz)],
        "nt_pair_block": [part, vp, vp, vp, P(NtBlockWeights), i32, i32, i32, ctypes.c_int, vp,
                          sz, vp],
        "nt_pair_block_noalloc": [part, vp, vp, vp, P(NtBlockWeights), i32, i32, i32,
                                  ctypes.c_int, vp],
        "nt_chain_workspace_bytes": [part, i32, i32, i32, i32, ctypes.c_int, P(sz)],
        "nt_pair_chain": [part, vp, vp, vp, P(NtBlockWeights), i32, i32, i32, i32, ctypes.c_int,
                          vp, sz, vp],
        "nt_pair_block_rect": [part, vp, vp, vp, vp, P(NtBlockWeights), i32, i32, i32,
                               ctypes.c_int, vp, sz, vp],
        "nt_pair_block_ex": [part, vp, vp, vp, vp, P(NtBlockParams), i32, i32, i32, ctypes.c_int,
                             vp, sz, vp],
        "nt_pair_chain_ex": [part, vp, vp, vp, P(NtBlockParams), i32, i32, i32, i32, ctypes.c_int,
                             vp, sz, vp],
        "nt_block_backward_ex_workspace_bytes": [part, i32, i32, i32, i32, ctypes.c_int, P(sz)],
        "nt_pair_block_backward_ex": [part, vp, vp, P(NtBlockParams), vp, vp, vp,
                                      P(NtBlockParamGrads), i32, i32, i32, ctypes.c_int, vp, sz,
                                      vp],
        "nt_loss_workspace_bytes": [part, P(sz)],
        "nt_pair_loss_eq5": [part, vp, i32, vp, i32, i32, ctypes.c_int, vp, vp, vp, vp, sz, vp],
        "nt_pair_reduce_backward": [part, vp, vp, vp, i32, vp],
        "nt_pair_broadcast_backward": [part, vp, vp, vp, i32, vp],
        "nt_transition_backward_workspace_bytes": [part, i32, i32, ctypes.c_int, P(sz)],
        "nt_pair_transition_backward": [part, vp, vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_int,
                                        vp, sz, vp],
        "nt_block_backward_workspace_bytes": [part, i32, i32, i32, ctypes.c_int, P(sz)],
        "nt_pair_block_backward": [part, vp, vp, P(NtBlockWeights), vp, vp, vp, P(NtBlockGrads),
                                   i32, i32, i32, ctypes.c_int, vp, sz, vp],
        "nt_block_nl_workspace_bytes": [part, i32, i32, i32, i32, ctypes.c_int, P(sz)],
        "nt_pair_block_nl": [part, vp, vp, vp, P(NtBlockWeights), i32, i32, i32, i32, ctypes.c_int,
                             vp, sz, vp],
        "nt_block_backward_nl_workspace_bytes": [part, i32, i32, i32, i32, ctypes.c_int, P(sz)],
        "nt_pair_block_backward_nl": [part, vp, vp, P(NtBlockWeights), vp, vp, vp, P(NtBlockGrads),
                                      i32, i32, i32, i32, ctypes.c_int, vp, sz, vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.nt_last_error.argtypes = []
    L.nt_last_error.restype = ctypes.c_char_p
    L.nt_version.argtypes = []
    L.nt_version.restype = ctypes.c_int32
    _lib = L
    return L
