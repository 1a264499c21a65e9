"""Packed single-pair-single block on MI355X: Python binding of libntpair.so.

The functions below carry the C entry points' names and only marshal
arguments: PyTorch supplies device memory and the current HIP stream, and
every step of the computation runs in the library's gfx950 kernels. There is
no fallback path; calls fail if the library is not built or rejects its
arguments (NtError carries the status and the library's message).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _native
from ._native import (NT_BF16, NT_F32, NT_TRANSITION_LN_SWIGLU,  # noqa: F401
                      NT_TRANSITION_RELU_MLP, NativeLibraryMissing, NtBlockParamGrads,
                      NtBlockParams, NtBlockWeights, NtPartition)

__all__ = ["NtError", "Partition", "nt_partition_sizes", "nt_make_partition",
           "nt_partition_sizes_rect", "nt_make_partition_rect", "nt_pair_block_rect",
           "nt_decode_cells",
           "nt_pair_broadcast", "nt_pair_transition", "nt_pair_broadcast_transition",
           "nt_pair_transition_swiglu", "nt_pair_reduce",
           "nt_block_workspace_bytes", "nt_pair_block", "nt_pair_block_noalloc",
           "nt_chain_workspace_bytes",
           "nt_pair_chain", "nt_pair_block_ex", "nt_pair_chain_ex", "nt_pair_block_backward_ex",
           "nt_block_backward_ex_workspace_bytes", "nt_last_error", "nt_version",
           "NT_F32", "NT_BF16"]


class NtError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_native.STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


def _check(status: int) -> None:
    if status != _native.NT_OK:
        raise NtError(status, _native.lib().nt_last_error().decode())


def nt_last_error() -> str:
    return _native.lib().nt_last_error().decode()


def nt_version() -> int:
    return int(_native.lib().nt_version())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return NT_BF16
    if t.dtype == torch.float32:
        return NT_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() if t.numel() else None


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _expect(p, name, t, shape, dtype=None):
    """Host-side extent check before a native call: the C ABI sees only
    pointers, so a tensor of the wrong shape or on another device would be
    read or written out of bounds by the kernels."""
    if t is None:
        return
    if t.device != p.device:
        raise ValueError(f"{name} is on {t.device}, the partition on {p.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _expect_workspace(p, workspace, need: int) -> None:
    if workspace.device != p.device:
        raise ValueError(f"workspace is on {workspace.device}, the partition on {p.device}")
    if _nbytes(workspace) < need:
        raise ValueError(f"workspace has {_nbytes(workspace)} bytes, needs {need}")


def _expect_weights(p, weights, c_s, c_z, hidden, dtype, label="") -> None:
    shapes = {"Wa": (c_z, c_s), "Wb": (c_z, c_s), "W1": (hidden, c_z), "W2": (c_z, hidden),
              "Wo": (c_s, c_z)}
    for name, w in zip(("Wa", "Wb", "W1", "W2", "Wo"), weights):
        _expect(p, label + name, w, shapes[name], dtype)


def _stream(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _lengths_array(lengths) -> np.ndarray:
    arr = np.ascontiguousarray(np.asarray(lengths, dtype=np.int64))
    if arr.ndim != 1:
        raise ValueError("lengths must be one-dimensional")
    if arr.size and (arr.min() < np.iinfo(np.int32).min or arr.max() > np.iinfo(np.int32).max):
        raise OverflowError("lengths must fit int32")
    return arr.astype(np.int32)


def nt_partition_sizes(lengths: Sequence[int]) -> Tuple[int, int, int, int]:
    """(T, cells, n_max, buffer_bytes) of a length vector; host only."""
    arr = _lengths_array(lengths)
    T, cells, n_max, nbytes = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32(), \
        ctypes.c_size_t()
    ptr = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if arr.size else None
    _check(_native.lib().nt_partition_sizes(ptr, arr.size, ctypes.byref(T), ctypes.byref(cells),
                                            ctypes.byref(n_max), ctypes.byref(nbytes)))
    return T.value, cells.value, n_max.value, nbytes.value


class Partition:
    """A built partition: the C struct plus the device buffer it points into."""

    def __init__(self, struct: NtPartition, buffer, lengths: np.ndarray):
        self.struct = struct
        self.buffer = buffer
        self.lengths = lengths

    B = property(lambda self: self.struct.B)
    T = property(lambda self: self.struct.T)
    T_cols = property(lambda self: self.struct.T_cols)
    rectangular = property(lambda self: self.struct.col_offsets != self.struct.single_offsets)
    cells = property(lambda self: self.struct.cells)
    n_max = property(lambda self: self.struct.n_max)
    n_items = property(lambda self: self.struct.n_items)
    device = property(lambda self: self.buffer.device)

    def _view(self, addr: int, count: int, dtype):
        torch = _torch()
        off = addr - self.buffer.data_ptr()
        size = torch.tensor([], dtype=dtype).element_size()
        return self.buffer[off:off + count * size].view(dtype)

    def arrays(self) -> dict:
        """Device views of the partition arrays (Figure 2's offsets and splits)."""
        torch = _torch()
        s, B, T = self.struct, self.B, self.T
        return {
            "lengths": self._view(s.lengths, B, torch.int32),
            "single_offsets": self._view(s.single_offsets, B + 1, torch.int64),
            "pair_offsets": self._view(s.pair_offsets, B + 1, torch.int64),
            "item_offsets": self._view(s.item_offsets, B + 1, torch.int64),
            "row_splits": self._view(s.row_splits, T + 1, torch.int64),
            "row_sample": self._view(s.row_sample, T, torch.int32),
            "tile_sample": self._view(s.tile_sample, (self.cells + 255) // 256, torch.int32),
            "col_lengths": self._view(s.col_lengths, B, torch.int32),
            "col_offsets": self._view(s.col_offsets, B + 1, torch.int64),
        }


def nt_make_partition(lengths, device=None, stream=None, buffer=None) -> Partition:
    """Build a square pair partition on the device (nt_make_partition).

    lengths: a sequence / numpy array (copied to pageable int32 memory), or a
    CPU int32 torch tensor, passed as is (if it is pinned, the copy to the
    device is asynchronous and the tensor must not change until the stream
    has passed the call). buffer: optional preallocated uint8 device tensor.
    """
    torch = _torch()
    host = None
    if isinstance(lengths, torch.Tensor):
        if lengths.device.type != "cpu" or lengths.dtype != torch.int32 or \
                not lengths.is_contiguous():
            raise ValueError("tensor lengths must be a contiguous CPU int32 tensor")
        host = lengths
        arr = lengths.numpy()
    else:
        arr = _lengths_array(lengths)
    _, _, _, nbytes = nt_partition_sizes(arr)
    dev = torch.device(device) if device is not None else torch.device("cuda",
                                                                        torch.cuda.current_device())
    if buffer is None or buffer.numel() < nbytes:
        buffer = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    st = NtPartition()
    ptr = ctypes.cast(host.data_ptr(), ctypes.POINTER(ctypes.c_int32)) if host is not None \
        else arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    if arr.size == 0:
        ptr = None
    _check(_native.lib().nt_make_partition(ptr, arr.size, buffer.data_ptr(), buffer.numel(),
                                           _stream(stream, dev), ctypes.byref(st)))
    return Partition(st, buffer, arr if host is None else host)


def nt_partition_sizes_rect(rows: Sequence[int], cols: Sequence[int]) -> Tuple[int, int, int, int]:
    """(T, T_cols, cells, buffer_bytes) of a rectangular partition; host only."""
    r, c = _lengths_array(rows), _lengths_array(cols)
    if r.size != c.size:
        raise ValueError("rows and cols must have one entry per sample")
    T, Tc, cells, nbytes = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    rp = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if r.size else None
    cp = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if c.size else None
    _check(_native.lib().nt_partition_sizes_rect(rp, cp, r.size, ctypes.byref(T), ctypes.byref(Tc),
                                                 ctypes.byref(cells), ctypes.byref(nbytes)))
    return T.value, Tc.value, cells.value, nbytes.value


def nt_make_partition_rect(rows, cols, device=None, stream=None, buffer=None) -> Partition:
    """Build a rectangular (N_i x M_i) pair partition on the device."""
    torch = _torch()
    r, c = _lengths_array(rows), _lengths_array(cols)
    _, _, _, nbytes = nt_partition_sizes_rect(r, c)
    dev = torch.device(device) if device is not None else torch.device("cuda",
                                                                        torch.cuda.current_device())
    if buffer is None or buffer.numel() < nbytes:
        buffer = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    st = NtPartition()
    rp = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if r.size else None
    cp = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if c.size else None
    _check(_native.lib().nt_make_partition_rect(rp, cp, r.size, buffer.data_ptr(), buffer.numel(),
                                                _stream(stream, dev), ctypes.byref(st)))
    part = Partition(st, buffer, r)
    part.col_lengths_host = c
    return part


def nt_decode_cells(p: Partition, stream=None):
    """(sample, row, col) int32 of every packed cell (test hook)."""
    torch = _torch()
    out = [torch.empty(p.cells, dtype=torch.int32, device=p.device) for _ in range(3)]
    _check(_native.lib().nt_decode_cells(ctypes.byref(p.struct), *[_ptr(t) for t in out],
                                         _stream(stream, p.device)))
    return tuple(out)


def nt_pair_broadcast(p: Partition, a, b, z=None, stream=None):
    """z[o_i + r N_i + c] = a[eta_i + r] + b[eta_i + c]."""
    torch = _torch()
    c_z = a.shape[-1]
    if z is None:
        z = torch.empty((p.cells, c_z), dtype=a.dtype, device=a.device)
    if a.dtype != b.dtype or z.dtype != a.dtype:
        raise TypeError("a, b and z must share a dtype")
    _expect(p, "a", a, (p.T, c_z))
    _expect(p, "b", b, (p.T_cols, c_z))
    _expect(p, "z", z, (p.cells, c_z))
    _check(_native.lib().nt_pair_broadcast(ctypes.byref(p.struct), _ptr(a), _ptr(b), _ptr(z),
                                           c_z, _dtype_code(a), _stream(stream, a.device)))
    return z


def nt_pair_transition(p: Partition, z_in, W1, W2, z_out=None, stream=None):
    """z_out = z_in + relu(z_in W1^T) W2^T; pass z_out=z_in to work in place."""
    torch = _torch()
    c_z, hidden = z_in.shape[-1], W1.shape[0]
    if z_out is None:
        z_out = torch.empty_like(z_in)
    if not (z_in.dtype == W1.dtype == W2.dtype == z_out.dtype):
        raise TypeError("z and weights must share a dtype")
    _expect(p, "z_in", z_in, (p.cells, c_z))
    _expect(p, "z_out", z_out, (p.cells, c_z))
    _expect(p, "W1", W1, (hidden, c_z))
    _expect(p, "W2", W2, (c_z, hidden))
    _check(_native.lib().nt_pair_transition(ctypes.byref(p.struct), _ptr(z_in), _ptr(z_out),
                                            _ptr(W1), _ptr(W2), c_z, hidden,
                                            _dtype_code(z_in), _stream(stream, z_in.device)))
    return z_out


def nt_pair_broadcast_transition(p: Partition, a, b, W1, W2, z_out=None, stream=None):
    """z_out = z + relu(z W1^T) W2^T with z = a[row] + b[col] formed on chip.

    a, b: float32 [T, c_z]; W1, W2 and z_out share the storage dtype.
    """
    torch = _torch()
    c_z, hidden = a.shape[-1], W1.shape[0]
    if a.dtype != torch.float32 or b.dtype != torch.float32:
        raise TypeError("a and b must be float32")
    if z_out is None:
        z_out = torch.empty((p.cells, c_z), dtype=W1.dtype, device=a.device)
    if not (W1.dtype == W2.dtype == z_out.dtype):
        raise TypeError("weights and z_out must share a dtype")
    _expect(p, "a", a, (p.T, c_z))
    _expect(p, "b", b, (p.T_cols, c_z))
    _expect(p, "z_out", z_out, (p.cells, c_z))
    _expect(p, "W1", W1, (hidden, c_z))
    _expect(p, "W2", W2, (c_z, hidden))
    _check(_native.lib().nt_pair_broadcast_transition(
        ctypes.byref(p.struct), _ptr(a), _ptr(b), _ptr(z_out), _ptr(W1), _ptr(W2), c_z, hidden,
        _dtype_code(W1), _stream(stream, a.device)))
    return z_out


def nt_pair_transition_swiglu(p: Partition, z_in, ln_gamma, ln_beta, W_gate, W_up, W_down,
                              z_out=None, ln_eps: float = 1e-5, stream=None):
    """z_out = z_in + (silu(x W_gate^T) * (x W_up^T)) W_down^T, x = LN(z_in).

    z_in, W_*: bf16; ln_gamma, ln_beta: float32 [c_z]; pass z_out=z_in to
    work in place.
    """
    torch = _torch()
    c_z, hidden = z_in.shape[-1], W_gate.shape[0]
    if z_out is None:
        z_out = torch.empty_like(z_in)
    if ln_gamma.dtype != torch.float32 or ln_beta.dtype != torch.float32:
        raise TypeError("ln_gamma and ln_beta must be float32")
    if not (z_in.dtype == W_gate.dtype == W_up.dtype == W_down.dtype == z_out.dtype):
        raise TypeError("z and weights must share a dtype")
    _expect(p, "z_in", z_in, (p.cells, c_z))
    _expect(p, "z_out", z_out, (p.cells, c_z))
    _expect(p, "ln_gamma", ln_gamma, (c_z,))
    _expect(p, "ln_beta", ln_beta, (c_z,))
    _expect(p, "W_gate", W_gate, (hidden, c_z))
    _expect(p, "W_up", W_up, (hidden, c_z))
    _expect(p, "W_down", W_down, (c_z, hidden))
    _check(_native.lib().nt_pair_transition_swiglu(
        ctypes.byref(p.struct), _ptr(z_in), _ptr(z_out), _ptr(ln_gamma), _ptr(ln_beta),
        _ptr(W_gate), _ptr(W_up), _ptr(W_down), c_z, hidden, ln_eps, _dtype_code(z_in),
        _stream(stream, z_in.device)))
    return z_out


def nt_pair_reduce(p: Partition, z, m=None, stream=None):
    """m[eta_i + r] = mean over columns c of z[o_i + r N_i + c] (fp32)."""
    torch = _torch()
    c_z = z.shape[-1]
    if m is None:
        m = torch.empty((p.T, c_z), dtype=torch.float32, device=z.device)
    _expect(p, "z", z, (p.cells, c_z))
    _expect(p, "m", m, (p.T, c_z), torch.float32)
    _check(_native.lib().nt_pair_reduce(ctypes.byref(p.struct), _ptr(z), _ptr(m), c_z,
                                        _dtype_code(z), _stream(stream, z.device)))
    return m


def nt_block_workspace_bytes(p: Partition, c_s: int, c_z: int, hidden: int, dtype) -> int:
    n = ctypes.c_size_t()
    code = dtype if isinstance(dtype, int) else (NT_BF16 if "bfloat16" in str(dtype) else NT_F32)
    _check(_native.lib().nt_block_workspace_bytes(ctypes.byref(p.struct), c_s, c_z, hidden, code,
                                                  ctypes.byref(n)))
    return n.value


def nt_pair_block(p: Partition, s_in, weights, s_out=None, z_out=None, workspace=None,
                  stream=None):
    """One single-pair-single block; returns (s_out, z_out).

    weights: dict (or sequence in this order) of Wa, Wb [c_z, c_s], W1
    [hidden, c_z], W2 [c_z, hidden], Wo [c_s, c_z], all in s_in's dtype.
    """
    torch = _torch()
    if isinstance(weights, dict):
        weights = [weights[k] for k in ("Wa", "Wb", "W1", "W2", "Wo")]
    Wa, Wb, W1, W2, Wo = weights
    c_s, c_z, hidden = s_in.shape[-1], Wa.shape[0], W1.shape[0]
    for w in weights:
        if w.dtype != s_in.dtype:
            raise TypeError("weights must share s_in's dtype")
    if s_out is None:
        s_out = torch.empty_like(s_in)
    if z_out is None:
        z_out = torch.empty((p.cells, c_z), dtype=s_in.dtype, device=s_in.device)
    need = nt_block_workspace_bytes(p, c_s, c_z, hidden, _dtype_code(s_in))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=s_in.device)
    _expect(p, "s_in", s_in, (p.T, c_s))
    _expect(p, "s_out", s_out, (p.T, c_s), s_in.dtype)
    _expect(p, "z_out", z_out, (p.cells, c_z), s_in.dtype)
    _expect_weights(p, weights, c_s, c_z, hidden, s_in.dtype)
    _expect_workspace(p, workspace, need)
    wst = NtBlockWeights(*[_ptr(w) for w in weights])
    _check(_native.lib().nt_pair_block(ctypes.byref(p.struct), _ptr(s_in), _ptr(s_out),
                                       _ptr(z_out), ctypes.byref(wst), c_s, c_z, hidden,
                                       _dtype_code(s_in), _ptr(workspace),
                                       _nbytes(workspace), _stream(stream, s_in.device)))
    return s_out, z_out


def nt_pair_block_noalloc(p: Partition, s_in, weights, s_out=None, z_out=None, stream=None):
    """nt_pair_block with its workspace in the library's static device
    scratch (nt_pair_block_noalloc): the native call allocates nothing.
    Pass s_out and z_out to keep this wrapper from allocating them."""
    torch = _torch()
    if isinstance(weights, dict):
        weights = [weights[k] for k in ("Wa", "Wb", "W1", "W2", "Wo")]
    Wa, Wb, W1, W2, Wo = weights
    c_s, c_z, hidden = s_in.shape[-1], Wa.shape[0], W1.shape[0]
    if s_out is None:
        s_out = torch.empty_like(s_in)
    if z_out is None:
        z_out = torch.empty((p.cells, c_z), dtype=s_in.dtype, device=s_in.device)
    _expect(p, "s_in", s_in, (p.T, c_s))
    _expect(p, "s_out", s_out, (p.T, c_s), s_in.dtype)
    _expect(p, "z_out", z_out, (p.cells, c_z), s_in.dtype)
    _expect_weights(p, weights, c_s, c_z, hidden, s_in.dtype)
    wst = NtBlockWeights(*[_ptr(w) for w in weights])
    _check(_native.lib().nt_pair_block_noalloc(ctypes.byref(p.struct), _ptr(s_in), _ptr(s_out),
                                               _ptr(z_out), ctypes.byref(wst), c_s, c_z, hidden,
                                               _dtype_code(s_in), _stream(stream, s_in.device)))
    return s_out, z_out


def nt_chain_workspace_bytes(p: Partition, nblocks: int, c_s: int, c_z: int, hidden: int,
                             dtype) -> int:
    n = ctypes.c_size_t()
    code = dtype if isinstance(dtype, int) else (NT_BF16 if "bfloat16" in str(dtype) else NT_F32)
    _check(_native.lib().nt_chain_workspace_bytes(ctypes.byref(p.struct), nblocks, c_s, c_z,
                                                  hidden, code, ctypes.byref(n)))
    return n.value


def nt_pair_chain(p: Partition, s_in, weights, s_out=None, z_out=None, workspace=None,
                  stream=None):
    """Blocks in sequence in one call; returns (s_out, z_out) of the last block.

    weights: a list with one entry per block, each as nt_pair_block takes it.
    """
    torch = _torch()
    sets = []
    for wk in weights:
        if isinstance(wk, dict):
            wk = [wk[k] for k in ("Wa", "Wb", "W1", "W2", "Wo")]
        for w in wk:
            if w.dtype != s_in.dtype:
                raise TypeError("weights must share s_in's dtype")
        sets.append(list(wk))
    if not sets:
        raise ValueError("at least one block")
    c_s, c_z, hidden = s_in.shape[-1], sets[0][0].shape[0], sets[0][2].shape[0]
    if s_out is None:
        s_out = torch.empty_like(s_in)
    if z_out is None:
        z_out = torch.empty((p.cells, c_z), dtype=s_in.dtype, device=s_in.device)
    need = nt_chain_workspace_bytes(p, len(sets), c_s, c_z, hidden, _dtype_code(s_in))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=s_in.device)
    _expect(p, "s_in", s_in, (p.T, c_s))
    _expect(p, "s_out", s_out, (p.T, c_s), s_in.dtype)
    _expect(p, "z_out", z_out, (p.cells, c_z), s_in.dtype)
    for k, wk in enumerate(sets):
        _expect_weights(p, wk, c_s, c_z, hidden, s_in.dtype, label=f"block {k} ")
    _expect_workspace(p, workspace, need)
    arr = (NtBlockWeights * len(sets))(*[NtBlockWeights(*[_ptr(w) for w in wk]) for wk in sets])
    _check(_native.lib().nt_pair_chain(ctypes.byref(p.struct), _ptr(s_in), _ptr(s_out),
                                       _ptr(z_out), arr, len(sets), c_s, c_z, hidden,
                                       _dtype_code(s_in), _ptr(workspace), _nbytes(workspace),
                                       _stream(stream, s_in.device)))
    return s_out, z_out


def nt_pair_block_rect(p: Partition, s_rows, s_cols, weights, s_out=None, z_out=None,
                       workspace=None, stream=None):
    """The rectangular block: pair rows from s_rows [T, c_s], columns from
    s_cols [T_cols, c_s]; returns (s_out, z_out)."""
    torch = _torch()
    if isinstance(weights, dict):
        weights = [weights[k] for k in ("Wa", "Wb", "W1", "W2", "Wo")]
    Wa, Wb, W1, W2, Wo = weights
    c_s, c_z, hidden = s_rows.shape[-1], Wa.shape[0], W1.shape[0]
    for w in weights:
        if w.dtype != s_rows.dtype:
            raise TypeError("weights must share s_rows' dtype")
    if s_cols.dtype != s_rows.dtype:
        raise TypeError("s_rows and s_cols must share a dtype")
    if s_out is None:
        s_out = torch.empty_like(s_rows)
    if z_out is None:
        z_out = torch.empty((p.cells, c_z), dtype=s_rows.dtype, device=s_rows.device)
    need = nt_block_workspace_bytes(p, c_s, c_z, hidden, _dtype_code(s_rows))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=s_rows.device)
    _expect(p, "s_rows", s_rows, (p.T, c_s))
    _expect(p, "s_cols", s_cols, (p.T_cols, c_s))
    _expect(p, "s_out", s_out, (p.T, c_s), s_rows.dtype)
    _expect(p, "z_out", z_out, (p.cells, c_z), s_rows.dtype)
    _expect_weights(p, weights, c_s, c_z, hidden, s_rows.dtype)
    _expect_workspace(p, workspace, need)
    wst = NtBlockWeights(*[_ptr(w) for w in weights])
    _check(_native.lib().nt_pair_block_rect(ctypes.byref(p.struct), _ptr(s_rows), _ptr(s_cols),
                                            _ptr(s_out), _ptr(z_out), ctypes.byref(wst), c_s, c_z,
                                            hidden, _dtype_code(s_rows), _ptr(workspace),
                                            _nbytes(workspace), _stream(stream, s_rows.device)))
    return s_out, z_out


# ------------------------------------------------------------------ backward
_WEIGHT_NAMES = ("Wa", "Wb", "W1", "W2", "Wo")


def _code(dtype) -> int:
    return dtype if isinstance(dtype, int) else (NT_BF16 if "bfloat16" in str(dtype) else NT_F32)


def nt_loss_workspace_bytes(p: Partition) -> int:
    n = ctypes.c_size_t()
    _check(_native.lib().nt_loss_workspace_bytes(ctypes.byref(p.struct), ctypes.byref(n)))
    return n.value


def nt_pair_loss_eq5(p: Partition, x, pz, S: int = 1, grads: bool = True, workspace=None,
                     stream=None):
    """Equation 5 over singles x [T, S*c_s] and pair state pz [cells, S*c_z]
    (S: the static axis of the non-leading layout, 1 for the leading one).
    Returns (loss, g_x, g_pz): loss a float64 device tensor of one element,
    the gradients fp32 (None when grads is False)."""
    torch = _torch()
    dev = x.device
    if pz.dtype != x.dtype:
        raise TypeError("x and pz must share a dtype")
    loss = torch.empty(2, dtype=torch.float64, device=dev)  # 16 bytes, aligned
    g_x = torch.empty(x.shape, dtype=torch.float32, device=dev) if grads else None
    g_pz = torch.empty(pz.shape, dtype=torch.float32, device=dev) if grads else None
    if workspace is None:
        workspace = torch.empty(nt_loss_workspace_bytes(p), dtype=torch.uint8, device=dev)
    if x.dim() != 2 or pz.dim() != 2 or x.shape[-1] % S or pz.shape[-1] % S:
        raise ValueError("x and pz must be 2-D with row widths that are multiples of S")
    _expect(p, "x", x, (p.T, x.shape[-1]))
    _expect(p, "pz", pz, (p.cells, pz.shape[-1]))
    _expect_workspace(p, workspace, nt_loss_workspace_bytes(p))
    _check(_native.lib().nt_pair_loss_eq5(ctypes.byref(p.struct), _ptr(x), x.shape[-1] // S,
                                          _ptr(pz), pz.shape[-1] // S, S, _dtype_code(x),
                                          _ptr(loss), _ptr(g_x),
                                          _ptr(g_pz), _ptr(workspace), _nbytes(workspace),
                                          _stream(stream, dev)))
    return loss[:1], g_x, g_pz


def nt_pair_reduce_backward(p: Partition, g_m, g_z_in=None, G=None, stream=None):
    """G = g_z_in (or 0) + g_m[row] / M_i on every cell (fp32)."""
    torch = _torch()
    c_z = g_m.shape[-1]
    if G is None:
        G = torch.empty((p.cells, c_z), dtype=torch.float32, device=g_m.device)
    _expect(p, "g_m", g_m, (p.T, c_z), torch.float32)
    _expect(p, "g_z_in", g_z_in, (p.cells, c_z), torch.float32)
    _expect(p, "G", G, (p.cells, c_z), torch.float32)
    _check(_native.lib().nt_pair_reduce_backward(ctypes.byref(p.struct), _ptr(g_m), _ptr(g_z_in),
                                                 _ptr(G), c_z, _stream(stream, g_m.device)))
    return G


def nt_pair_broadcast_backward(p: Partition, g_z, g_a=None, g_b=None, stream=None):
    """Row sums g_a [T, c_z] and column sums g_b [T_cols, c_z] of g_z (fp32)."""
    torch = _torch()
    c_z = g_z.shape[-1]
    if g_a is None:
        g_a = torch.empty((p.T, c_z), dtype=torch.float32, device=g_z.device)
    if g_b is None:
        g_b = torch.empty((p.T_cols, c_z), dtype=torch.float32, device=g_z.device)
    _expect(p, "g_z", g_z, (p.cells, c_z), torch.float32)
    _expect(p, "g_a", g_a, (p.T, c_z), torch.float32)
    _expect(p, "g_b", g_b, (p.T_cols, c_z), torch.float32)
    _check(_native.lib().nt_pair_broadcast_backward(ctypes.byref(p.struct), _ptr(g_z), _ptr(g_a),
                                                    _ptr(g_b), c_z, _stream(stream, g_z.device)))
    return g_a, g_b


def nt_transition_backward_workspace_bytes(p: Partition, c_z: int, hidden: int, dtype) -> int:
    n = ctypes.c_size_t()
    _check(_native.lib().nt_transition_backward_workspace_bytes(
        ctypes.byref(p.struct), c_z, hidden, _code(dtype), ctypes.byref(n)))
    return n.value


def nt_pair_transition_backward(p: Partition, z, G, W1, W2, g_z=None, dW1=None, dW2=None,
                                workspace=None, stream=None):
    """Gradient of z + relu(z W1^T) W2^T for G = dL/dz' (fp32). Returns
    (g_z, dW1, dW2), all fp32; g_z may be G (in place)."""
    torch = _torch()
    dev = z.device
    c_z, hidden = z.shape[-1], W1.shape[0]
    f32 = torch.float32
    if g_z is None:
        g_z = torch.empty((p.cells, c_z), dtype=f32, device=dev)
    if dW1 is None:
        dW1 = torch.empty((hidden, c_z), dtype=f32, device=dev)
    if dW2 is None:
        dW2 = torch.empty((c_z, hidden), dtype=f32, device=dev)
    need = nt_transition_backward_workspace_bytes(p, c_z, hidden, _dtype_code(z))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _expect(p, "z", z, (p.cells, c_z))
    _expect(p, "G", G, (p.cells, c_z), f32)
    _expect(p, "W1", W1, (hidden, c_z), z.dtype)
    _expect(p, "W2", W2, (c_z, hidden), z.dtype)
    _expect(p, "g_z", g_z, (p.cells, c_z), f32)
    _expect(p, "dW1", dW1, (hidden, c_z), f32)
    _expect(p, "dW2", dW2, (c_z, hidden), f32)
    _expect_workspace(p, workspace, need)
    _check(_native.lib().nt_pair_transition_backward(
        ctypes.byref(p.struct), _ptr(z), _ptr(G), _ptr(W1), _ptr(W2), _ptr(g_z), _ptr(dW1),
        _ptr(dW2), c_z, hidden, _dtype_code(z), _ptr(workspace), _nbytes(workspace),
        _stream(stream, dev)))
    return g_z, dW1, dW2


def nt_block_backward_workspace_bytes(p: Partition, c_s: int, c_z: int, hidden: int,
                                      dtype) -> int:
    n = ctypes.c_size_t()
    _check(_native.lib().nt_block_backward_workspace_bytes(ctypes.byref(p.struct), c_s, c_z,
                                                           hidden, _code(dtype),
                                                           ctypes.byref(n)))
    return n.value


def nt_pair_block_backward(p: Partition, s_in, z_out, weights, g_s_out, g_z_out=None,
                           g_s_in=None, grads=None, workspace=None, stream=None):
    """Backward of nt_pair_block: s_in and z_out are the block's input singles
    and returned pair state, g_s_out (and optionally g_z_out) the incoming
    fp32 gradients. Returns (g_s_in, grads) with grads a dict of fp32 weight
    gradients keyed like the weights."""
    torch = _torch()
    dev = s_in.device
    if isinstance(weights, dict):
        weights = [weights[k] for k in _WEIGHT_NAMES]
    Wa, Wb, W1, W2, Wo = weights
    c_s, c_z, hidden = s_in.shape[-1], Wa.shape[0], W1.shape[0]
    for w in weights:
        if w.dtype != s_in.dtype:
            raise TypeError("weights must share s_in's dtype")
    if g_s_in is None:
        g_s_in = torch.empty((p.T, c_s), dtype=torch.float32, device=dev)
    if grads is None:
        grads = {k: torch.empty(w.shape, dtype=torch.float32, device=dev)
                 for k, w in zip(_WEIGHT_NAMES, weights)}
    need = nt_block_backward_workspace_bytes(p, c_s, c_z, hidden, _dtype_code(s_in))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    f32 = torch.float32
    _expect(p, "s_in", s_in, (p.T, c_s))
    _expect(p, "z_out", z_out, (p.cells, c_z), s_in.dtype)
    _expect_weights(p, weights, c_s, c_z, hidden, s_in.dtype)
    _expect(p, "g_s_out", g_s_out, (p.T, c_s), f32)
    _expect(p, "g_z_out", g_z_out, (p.cells, c_z), f32)
    _expect(p, "g_s_in", g_s_in, (p.T, c_s), f32)
    _expect_weights(p, [grads[k] for k in _WEIGHT_NAMES], c_s, c_z, hidden, f32, label="d")
    _expect_workspace(p, workspace, need)
    wst = NtBlockWeights(*[_ptr(w) for w in weights])
    gst = _native.NtBlockGrads(*[_ptr(grads[k]) for k in _WEIGHT_NAMES])
    _check(_native.lib().nt_pair_block_backward(
        ctypes.byref(p.struct), _ptr(s_in), _ptr(z_out), ctypes.byref(wst), _ptr(g_s_out),
        _ptr(g_z_out), _ptr(g_s_in), ctypes.byref(gst), c_s, c_z, hidden, _dtype_code(s_in),
        _ptr(workspace), _nbytes(workspace), _stream(stream, dev)))
    return g_s_in, grads


# ------------------------------------------------------ non-leading layout
def nt_block_nl_workspace_bytes(p: Partition, S: int, c_s: int, c_z: int, hidden: int,
                                dtype) -> int:
    n = ctypes.c_size_t()
    _check(_native.lib().nt_block_nl_workspace_bytes(ctypes.byref(p.struct), S, c_s, c_z, hidden,
                                                     _code(dtype), ctypes.byref(n)))
    return n.value


def nt_block_backward_nl_workspace_bytes(p: Partition, S: int, c_s: int, c_z: int, hidden: int,
                                         dtype) -> int:
    n = ctypes.c_size_t()
    _check(_native.lib().nt_block_backward_nl_workspace_bytes(
        ctypes.byref(p.struct), S, c_s, c_z, hidden, _code(dtype), ctypes.byref(n)))
    return n.value


def nt_pair_block_nl(p: Partition, s_in, weights, S: int, s_out=None, z_out=None,
                     workspace=None, stream=None):
    """The block on the non-leading layout: s_in [T, S*c_s]; returns
    (s_out [T, S*c_s], z_out [cells, S*c_z])."""
    torch = _torch()
    if isinstance(weights, dict):
        weights = [weights[k] for k in _WEIGHT_NAMES]
    Wa, Wb, W1, W2, Wo = weights
    c_s, c_z, hidden = Wa.shape[1], Wa.shape[0], W1.shape[0]
    if s_in.shape[-1] != S * c_s:
        raise ValueError("s_in rows must hold S * c_s values")
    if s_out is None:
        s_out = torch.empty_like(s_in)
    if z_out is None:
        z_out = torch.empty((p.cells, S * c_z), dtype=s_in.dtype, device=s_in.device)
    need = nt_block_nl_workspace_bytes(p, S, c_s, c_z, hidden, _dtype_code(s_in))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=s_in.device)
    _expect(p, "s_in", s_in, (p.T, S * c_s))
    _expect(p, "s_out", s_out, (p.T, S * c_s), s_in.dtype)
    _expect(p, "z_out", z_out, (p.cells, S * c_z), s_in.dtype)
    _expect_weights(p, weights, c_s, c_z, hidden, s_in.dtype)
    _expect_workspace(p, workspace, need)
    wst = NtBlockWeights(*[_ptr(w) for w in weights])
    _check(_native.lib().nt_pair_block_nl(ctypes.byref(p.struct), _ptr(s_in), _ptr(s_out),
                                          _ptr(z_out), ctypes.byref(wst), S, c_s, c_z, hidden,
                                          _dtype_code(s_in), _ptr(workspace), _nbytes(workspace),
                                          _stream(stream, s_in.device)))
    return s_out, z_out


def nt_pair_block_backward_nl(p: Partition, s_in, z_out, weights, S: int, g_s_out, g_z_out=None,
                              g_s_in=None, grads=None, workspace=None, stream=None):
    """Backward of nt_pair_block_nl; returns (g_s_in, grads)."""
    torch = _torch()
    dev = s_in.device
    if isinstance(weights, dict):
        weights = [weights[k] for k in _WEIGHT_NAMES]
    Wa, Wb, W1, W2, Wo = weights
    c_s, c_z, hidden = Wa.shape[1], Wa.shape[0], W1.shape[0]
    if g_s_in is None:
        g_s_in = torch.empty((p.T, S * c_s), dtype=torch.float32, device=dev)
    if grads is None:
        grads = {k: torch.empty(w.shape, dtype=torch.float32, device=dev)
                 for k, w in zip(_WEIGHT_NAMES, weights)}
    need = nt_block_backward_nl_workspace_bytes(p, S, c_s, c_z, hidden, _dtype_code(s_in))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    f32 = torch.float32
    _expect(p, "s_in", s_in, (p.T, S * c_s))
    _expect(p, "z_out", z_out, (p.cells, S * c_z), s_in.dtype)
    _expect_weights(p, weights, c_s, c_z, hidden, s_in.dtype)
    _expect(p, "g_s_out", g_s_out, (p.T, S * c_s), f32)
    _expect(p, "g_z_out", g_z_out, (p.cells, S * c_z), f32)
    _expect(p, "g_s_in", g_s_in, (p.T, S * c_s), f32)
    _expect_weights(p, [grads[k] for k in _WEIGHT_NAMES], c_s, c_z, hidden, f32, label="d")
    _expect_workspace(p, workspace, need)
    wst = NtBlockWeights(*[_ptr(w) for w in weights])
    gst = _native.NtBlockGrads(*[_ptr(grads[k]) for k in _WEIGHT_NAMES])
    _check(_native.lib().nt_pair_block_backward_nl(
        ctypes.byref(p.struct), _ptr(s_in), _ptr(z_out), ctypes.byref(wst), _ptr(g_s_out),
        _ptr(g_z_out), _ptr(g_s_in), ctypes.byref(gst), S, c_s, c_z, hidden, _dtype_code(s_in),
        _ptr(workspace), _nbytes(workspace), _stream(stream, dev)))
    return g_s_in, grads


# ------------------------------------------- blocks with a named transition
_KIND_KEYS = {NT_TRANSITION_RELU_MLP: ("Wa", "Wb", "Wo", "W1", "W2"),
              NT_TRANSITION_LN_SWIGLU: ("Wa", "Wb", "Wo", "ln_gamma", "ln_beta", "W_gate", "W_up",
                                        "W_down")}


def _kind_of(params: dict) -> int:
    """NT_TRANSITION_LN_SWIGLU when the parameters hold W_gate, else the ReLU MLP."""
    return NT_TRANSITION_LN_SWIGLU if "W_gate" in params else NT_TRANSITION_RELU_MLP


def _expect_params(p, params: dict, c_s, c_z, hidden, dtype, label="") -> int:
    torch = _torch()
    kind = _kind_of(params)
    shapes = {"Wa": (c_z, c_s), "Wb": (c_z, c_s), "Wo": (c_s, c_z), "W1": (hidden, c_z),
              "W2": (c_z, hidden), "ln_gamma": (c_z,), "ln_beta": (c_z,),
              "W_gate": (hidden, c_z), "W_up": (hidden, c_z), "W_down": (c_z, hidden)}
    for k in _KIND_KEYS[kind]:
        if k not in params:
            raise KeyError(f"{label}{k} missing")
        dt = torch.float32 if k.startswith("ln_") else dtype
        _expect(p, label + k, params[k], shapes[k], dt)
    return kind


def _params_struct(params: dict, ln_eps: float) -> NtBlockParams:
    st = NtBlockParams()
    st.kind = _kind_of(params)
    st.ln_eps = ln_eps
    for k in _KIND_KEYS[st.kind]:
        setattr(st, k, _ptr(params[k]))
    return st


def _widths(params: dict):
    kind = _kind_of(params)
    c_z, c_s = params["Wa"].shape
    hidden = params["W1" if kind == NT_TRANSITION_RELU_MLP else "W_gate"].shape[0]
    return c_s, c_z, hidden


def nt_pair_block_ex(p: Partition, s_in, params: dict, s_cols=None, s_out=None, z_out=None,
                     workspace=None, ln_eps: float = 1e-5, stream=None):
    """One block with its transition named by its parameters: Wa, Wb, Wo
    and either W1, W2 (the ReLU MLP) or ln_gamma, ln_beta (fp32), W_gate,
    W_up, W_down (the pre-normalised SwiGLU). Returns (s_out, z_out)."""
    torch = _torch()
    c_s, c_z, hidden = _widths(params)
    if s_out is None:
        s_out = torch.empty_like(s_in)
    if z_out is None:
        z_out = torch.empty((p.cells, c_z), dtype=s_in.dtype, device=s_in.device)
    need = nt_block_workspace_bytes(p, c_s, c_z, hidden, _dtype_code(s_in))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=s_in.device)
    _expect(p, "s_in", s_in, (p.T, c_s))
    _expect(p, "s_cols", s_cols, (p.T_cols, c_s), s_in.dtype)
    _expect(p, "s_out", s_out, (p.T, c_s), s_in.dtype)
    _expect(p, "z_out", z_out, (p.cells, c_z), s_in.dtype)
    _expect_params(p, params, c_s, c_z, hidden, s_in.dtype)
    _expect_workspace(p, workspace, need)
    st = _params_struct(params, ln_eps)
    _check(_native.lib().nt_pair_block_ex(ctypes.byref(p.struct), _ptr(s_in), _ptr(s_cols),
                                          _ptr(s_out), _ptr(z_out), ctypes.byref(st), c_s, c_z,
                                          hidden, _dtype_code(s_in), _ptr(workspace),
                                          _nbytes(workspace), _stream(stream, s_in.device)))
    return s_out, z_out


def nt_pair_chain_ex(p: Partition, s_in, params: list, s_out=None, z_out=None, workspace=None,
                     ln_eps: float = 1e-5, stream=None):
    """Blocks in sequence, each with the parameters nt_pair_block_ex takes;
    returns (s_out, z_out) of the last block."""
    torch = _torch()
    if not params:
        raise ValueError("at least one block")
    c_s, c_z, hidden = _widths(params[0])
    if s_out is None:
        s_out = torch.empty_like(s_in)
    if z_out is None:
        z_out = torch.empty((p.cells, c_z), dtype=s_in.dtype, device=s_in.device)
    need = nt_chain_workspace_bytes(p, len(params), c_s, c_z, hidden, _dtype_code(s_in))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=s_in.device)
    _expect(p, "s_in", s_in, (p.T, c_s))
    _expect(p, "s_out", s_out, (p.T, c_s), s_in.dtype)
    _expect(p, "z_out", z_out, (p.cells, c_z), s_in.dtype)
    for k, pk in enumerate(params):
        _expect_params(p, pk, c_s, c_z, hidden, s_in.dtype, label=f"block {k} ")
    _expect_workspace(p, workspace, need)
    arr = (NtBlockParams * len(params))(*[_params_struct(pk, ln_eps) for pk in params])
    _check(_native.lib().nt_pair_chain_ex(ctypes.byref(p.struct), _ptr(s_in), _ptr(s_out),
                                          _ptr(z_out), arr, len(params), c_s, c_z, hidden,
                                          _dtype_code(s_in), _ptr(workspace), _nbytes(workspace),
                                          _stream(stream, s_in.device)))
    return s_out, z_out


def nt_block_backward_ex_workspace_bytes(p: Partition, kind: int, c_s: int, c_z: int,
                                         hidden: int, dtype) -> int:
    n = ctypes.c_size_t()
    _check(_native.lib().nt_block_backward_ex_workspace_bytes(
        ctypes.byref(p.struct), kind, c_s, c_z, hidden, _code(dtype), ctypes.byref(n)))
    return n.value


def nt_pair_block_backward_ex(p: Partition, s_in, z_out, params: dict, g_s_out, g_z_out=None,
                              g_s_in=None, grads=None, workspace=None, ln_eps: float = 1e-5,
                              stream=None):
    """Backward of nt_pair_block_ex; returns (g_s_in, grads), grads a dict of
    fp32 gradients keyed like the kind's parameters."""
    torch = _torch()
    dev = s_in.device
    kind = _kind_of(params)
    c_s, c_z, hidden = _widths(params)
    f32 = torch.float32
    if g_s_in is None:
        g_s_in = torch.empty((p.T, c_s), dtype=f32, device=dev)
    if grads is None:
        grads = {k: torch.empty(params[k].shape, dtype=f32, device=dev) for k in _KIND_KEYS[kind]}
    need = nt_block_backward_ex_workspace_bytes(p, kind, c_s, c_z, hidden, _dtype_code(s_in))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _expect(p, "s_in", s_in, (p.T, c_s))
    _expect(p, "z_out", z_out, (p.cells, c_z), s_in.dtype)
    _expect_params(p, params, c_s, c_z, hidden, s_in.dtype)
    _expect(p, "g_s_out", g_s_out, (p.T, c_s), f32)
    _expect(p, "g_z_out", g_z_out, (p.cells, c_z), f32)
    _expect(p, "g_s_in", g_s_in, (p.T, c_s), f32)
    for k in _KIND_KEYS[kind]:
        _expect(p, "d" + k, grads[k], tuple(params[k].shape), f32)
    _expect_workspace(p, workspace, need)
    st = _params_struct(params, ln_eps)
    gst = NtBlockParamGrads()
    for k in _KIND_KEYS[kind]:
        setattr(gst, k, _ptr(grads[k]))
    _check(_native.lib().nt_pair_block_backward_ex(
        ctypes.byref(p.struct), _ptr(s_in), _ptr(z_out), ctypes.byref(st), _ptr(g_s_out),
        _ptr(g_z_out), _ptr(g_s_in), ctypes.byref(gst), c_s, c_z, hidden, _dtype_code(s_in),
        _ptr(workspace), _nbytes(workspace), _stream(stream, dev)))
    return g_s_in, grads
