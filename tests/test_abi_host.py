"""Host-side checks of the C ABI (no GPU needed).

The library must load and export every function include/nt_pair.h declares,
size partitions like the oracle, and reject invalid arguments with the right
status before anything is enqueued. No call here reaches a HIP launch: each
argument set is invalid by construction.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from padding_free_pair_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nt_pair.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_native.LIB_PATH):
        from padding_free_pair_amd import build
        build.build(verbose=False)
    return _native.lib()


def declared_functions():
    text = open(HEADER).read()
    return set(re.findall(r"^\s*(?:nt_status|const char\s*\*|int32_t)\s+(nt_\w+)\s*\(", text,
                          flags=re.M))


def test_header_and_binding_agree():
    assert declared_functions() == set(_native.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _native.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = declared_functions() - exported
    assert not missing, missing
    for name in declared_functions():
        assert hasattr(lib, name)
    assert lib.nt_version() == 1


def test_struct_layout_matches_header(lib):
    # int32 x4, int64 x3, seven pointers, then T_cols and two more pointers
    assert ctypes.sizeof(_native.NtPartition) == 16 + 24 + 7 * 8 + 8 + 2 * 8
    assert _native.NtPartition.lengths.offset == 40
    assert ctypes.sizeof(_native.NtBlockWeights) == 5 * 8


def _sizes(lib, lengths):
    arr = np.ascontiguousarray(lengths, dtype=np.int32)
    T, cells, nmax, nb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_size_t()
    ptr = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if arr.size else None
    st = lib.nt_partition_sizes(ptr, arr.size, ctypes.byref(T), ctypes.byref(cells),
                                ctypes.byref(nmax), ctypes.byref(nb))
    return st, T.value, cells.value, nmax.value, nb.value


@pytest.mark.parametrize("lengths", [[2, 3], [7, 12, 5, 16], [0], [], [0, 0, 9, 0],
                                     [1024, 768, 384, 96], list(range(300))])
def test_partition_sizes_match_oracle(lib, lengths):
    st, T, cells, nmax, nb = _sizes(lib, lengths)
    p = oracle.partition(lengths)
    assert st == 0
    assert (T, cells, nmax) == (p["T"], p["cells"], p["n_max"])
    assert nb >= 8 * (len(lengths) + 1) * 3 + 8 * (T + 1) + 4 * T


def test_partition_sizes_errors(lib):
    assert _sizes(lib, [3, -1])[0] == _native.NT_ERR_INVALID
    assert "negative" in lib.nt_last_error().decode()
    # sum of squares beyond the cell limit
    assert _sizes(lib, [2 ** 31 - 1])[0] == _native.NT_ERR_OVERFLOW
    # T beyond int32
    assert _sizes(lib, [2 ** 30] * 3)[0] == _native.NT_ERR_OVERFLOW
    assert lib.nt_partition_sizes(None, 2, None, None, None, None) == _native.NT_ERR_NULL
    assert lib.nt_partition_sizes(None, -1, None, None, None, None) == _native.NT_ERR_INVALID
    assert lib.nt_partition_sizes(None, 0, None, None, None, None) == _native.NT_OK


def test_make_partition_rejects_before_launch(lib):
    arr = np.array([2, 3], dtype=np.int32)
    ptr = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    out = _native.NtPartition()
    need = _sizes(lib, [2, 3])[4]
    assert lib.nt_make_partition(ptr, 2, None, need, None, ctypes.byref(out)) == _native.NT_ERR_NULL
    assert lib.nt_make_partition(ptr, 2, 0x10000 + 64, need, None,
                                 ctypes.byref(out)) == _native.NT_ERR_ALIGN
    assert lib.nt_make_partition(ptr, 2, 0x10000, need - 1, None,
                                 ctypes.byref(out)) == _native.NT_ERR_WORKSPACE
    assert lib.nt_make_partition(ptr, 2, 0x10000, need, None, None) == _native.NT_ERR_NULL
    bad = np.array([2, -3], dtype=np.int32)
    assert lib.nt_make_partition(bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2, 0x10000,
                                 need, None, ctypes.byref(out)) == _native.NT_ERR_INVALID
    assert out.magic == 0  # untouched on failure


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation


def fake_partition(B=2, T=5, cells=13):
    p = _native.NtPartition()
    p.magic = 0x4E545031
    p.B, p.T, p.cells, p.n_items, p.n_max = B, T, cells, 2, 3
    for k, name in enumerate(("lengths", "single_offsets", "pair_offsets", "row_splits",
                              "row_sample", "item_offsets", "tile_sample")):
        setattr(p, name, FAKE + 0x1000 * k)
    p.T_cols, p.col_lengths, p.col_offsets = T, p.lengths, p.single_offsets
    return p


def test_stage_calls_validate(lib):
    p = fake_partition()
    P = ctypes.byref(p)
    a, b, z = FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000
    E = _native
    # unbuilt partition
    raw = _native.NtPartition()
    assert lib.nt_pair_broadcast(ctypes.byref(raw), a, b, z, 16, 1, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_broadcast(None, a, b, z, 16, 1, None) == E.NT_ERR_NULL
    # widths
    for cz in (0, 12, -8, 520):
        assert lib.nt_pair_broadcast(P, a, b, z, cz, 1, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_broadcast(P, a, b, z, 16, 7, None) == E.NT_ERR_DTYPE
    assert lib.nt_pair_broadcast(P, None, b, z, 16, 1, None) == E.NT_ERR_NULL
    assert lib.nt_pair_broadcast(P, a + 8, b, z, 16, 1, None) == E.NT_ERR_ALIGN
    # z overlapping b
    assert lib.nt_pair_broadcast(P, a, b, b + 16, 16, 1, None) == E.NT_ERR_INVALID
    # transition
    W1, W2 = FAKE + 0x400000, FAKE + 0x500000
    assert lib.nt_pair_transition(P, z, z, W1, W2, 16, 12, 1, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_transition(P, z, z + 32, W1, W2, 16, 32, 1, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_transition(P, z, W1 + 16, W1, W2, 16, 32, 1, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_transition(P, z, z, None, W2, 16, 32, 1, None) == E.NT_ERR_NULL
    # reduce
    assert lib.nt_pair_reduce(P, z, None, 16, 1, None) == E.NT_ERR_NULL
    assert lib.nt_pair_reduce(P, z, z + 16, 16, 1, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_reduce(P, z, a + 4, 16, 1, None) == E.NT_ERR_ALIGN
    # decode
    assert lib.nt_decode_cells(P, None, a, b, None) == E.NT_ERR_NULL
    # SwiGLU transition: bf16 only, c_z 64 or 128, hidden a multiple of 32
    g, bt, Wg, Wu, Wd = (FAKE + 0x600000 + 0x10000 * k for k in range(5))
    sw = lib.nt_pair_transition_swiglu
    assert sw(P, z, z, g, bt, Wg, Wu, Wd, 128, 512, 1e-5, 0, None) == E.NT_ERR_DTYPE
    assert sw(P, z, z, g, bt, Wg, Wu, Wd, 96, 512, 1e-5, 1, None) == E.NT_ERR_INVALID
    assert sw(P, z, z, g, bt, Wg, Wu, Wd, 128, 48, 1e-5, 1, None) == E.NT_ERR_INVALID
    assert sw(P, z, z, g, bt, Wg, Wu, Wd, 128, 512, -1.0, 1, None) == E.NT_ERR_INVALID
    assert sw(P, z, z, g, bt, Wg, Wu, Wd, 128, 512, float("nan"), 1, None) == E.NT_ERR_INVALID
    assert sw(P, z, z, None, bt, Wg, Wu, Wd, 128, 512, 1e-5, 1, None) == E.NT_ERR_NULL
    assert sw(P, z, z, g, bt, Wg, None, Wd, 128, 512, 1e-5, 1, None) == E.NT_ERR_NULL
    assert sw(P, z, z + 64, g, bt, Wg, Wu, Wd, 128, 512, 1e-5, 1, None) == E.NT_ERR_INVALID
    assert sw(P, z, Wd, g, bt, Wg, Wu, Wd, 128, 512, 1e-5, 1, None) == E.NT_ERR_INVALID
    assert sw(P, z, z, g + 4, bt, Wg, Wu, Wd, 128, 512, 1e-5, 1, None) == E.NT_ERR_ALIGN


def test_block_validates(lib):
    p = fake_partition()
    P = ctypes.byref(p)
    s, so, z = FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000
    w = _native.NtBlockWeights(FAKE + 0x400000, FAKE + 0x410000, FAKE + 0x420000,
                               FAKE + 0x430000, FAKE + 0x440000)
    ws = FAKE + 0x800000
    need = ctypes.c_size_t()
    assert lib.nt_block_workspace_bytes(P, 16, 16, 32, 1, ctypes.byref(need)) == 0
    assert need.value >= 2 * 5 * 16 * 2 + 5 * 16 * 4
    E = _native
    W = ctypes.byref(w)
    assert lib.nt_pair_block(P, s, so, z, W, 16, 16, 32, 1, ws, need.value - 1,
                             None) == E.NT_ERR_WORKSPACE
    assert lib.nt_pair_block(P, s, so, z, W, 16, 16, 32, 1, None, need.value,
                             None) == E.NT_ERR_NULL
    assert lib.nt_pair_block(P, s, so, z, None, 16, 16, 32, 1, ws, need.value,
                             None) == E.NT_ERR_NULL
    assert lib.nt_pair_block(P, s, s + 16, z, W, 16, 16, 32, 1, ws, need.value,
                             None) == E.NT_ERR_INVALID
    assert lib.nt_pair_block(P, s, so, ws, W, 16, 16, 32, 1, ws, need.value,
                             None) == E.NT_ERR_INVALID
    assert lib.nt_pair_block(P, s, so, z, W, 20, 16, 32, 1, ws, need.value,
                             None) == E.NT_ERR_INVALID
    w.W1 = None
    assert lib.nt_pair_block(P, s, so, z, W, 16, 16, 32, 1, ws, need.value,
                             None) == E.NT_ERR_NULL


def _sizes_rect(lib, rows, cols):
    r = np.ascontiguousarray(rows, dtype=np.int32)
    c = np.ascontiguousarray(cols, dtype=np.int32)
    T, Tc, cells, nb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    rp = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if r.size else None
    cp = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if c.size else None
    st = lib.nt_partition_sizes_rect(rp, cp, r.size, ctypes.byref(T), ctypes.byref(Tc),
                                     ctypes.byref(cells), ctypes.byref(nb))
    return st, T.value, Tc.value, cells.value, nb.value


@pytest.mark.parametrize("rows,cols", [([2, 0, 3], [4, 5, 1]), ([7, 12], [7, 12]), ([], []),
                                       ([0, 9], [3, 0])])
def test_rect_partition_sizes_match_oracle(lib, rows, cols):
    st, T, Tc, cells, nb = _sizes_rect(lib, rows, cols)
    assert st == _native.NT_OK
    ref = oracle.partition_rect(rows, cols)
    assert (T, Tc, cells) == (ref["T"], ref["T_cols"], ref["cells"])
    assert nb >= 256


def test_rect_partition_sizes_errors(lib):
    assert _sizes_rect(lib, [3, 2], [1, -1])[0] == _native.NT_ERR_INVALID
    assert _sizes_rect(lib, [2 ** 30, 2 ** 30], [1, 1])[0] == _native.NT_ERR_OVERFLOW  # T > 2^31 - 1
    assert _sizes_rect(lib, [2 ** 29, 2 ** 29], [1, 1])[0] == _native.NT_OK
    assert _sizes_rect(lib, [1], [2 ** 31 - 1])[0] == _native.NT_OK
    assert _sizes_rect(lib, [2 ** 31 - 1], [2 ** 31 - 1])[0] == _native.NT_ERR_OVERFLOW
    out = _native.NtPartition()
    r = np.array([2, 3], dtype=np.int32)
    rp = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.nt_make_partition_rect(rp, None, 2, 0x10000, 1 << 20, None,
                                      ctypes.byref(out)) == _native.NT_ERR_NULL


def test_square_block_rejects_rect_partition(lib):
    p = fake_partition()
    p.col_offsets = FAKE + 0x9000  # a rectangular partition's own column offsets
    P = ctypes.byref(p)
    w = _native.NtBlockWeights(*[FAKE + 0x100000 * (k + 1) for k in range(5)])
    s, z, ws = FAKE + 0x800000, FAKE + 0x900000, FAKE + 0xA00000
    assert lib.nt_pair_block(P, s, s, z, ctypes.byref(w), 16, 16, 32, 1, ws, 1 << 20,
                             None) == _native.NT_ERR_INVALID
    assert "nt_pair_block_rect" in lib.nt_last_error().decode()


def test_backward_calls_validate(lib):
    p = fake_partition()
    P = ctypes.byref(p)
    E = _native
    x, pz, loss, gx, gp, ws = (FAKE + 0x100000 * (k + 1) for k in range(6))
    need = ctypes.c_size_t()
    assert lib.nt_loss_workspace_bytes(P, ctypes.byref(need)) == 0
    assert need.value >= 5 * 8
    lw = need.value
    assert lib.nt_pair_loss_eq5(P, x, 16, pz, 16, 0, 1, loss, gx, gp, ws, lw, None) == \
        E.NT_ERR_INVALID                                                   # S < 1
    assert lib.nt_pair_loss_eq5(P, x, 16, pz, 16, 1, 1, None, gx, gp, ws, lw, None) == \
        E.NT_ERR_NULL
    assert lib.nt_pair_loss_eq5(P, x, 16, pz, 16, 1, 1, loss, gx, gp, ws, lw - 1, None) == \
        E.NT_ERR_WORKSPACE
    assert lib.nt_pair_loss_eq5(P, x, 16, pz, 16, 1, 1, loss, x + 16, gp, ws, lw, None) == \
        E.NT_ERR_INVALID                                                   # g_x overlaps x
    assert lib.nt_pair_loss_eq5(P, x, 12, pz, 16, 1, 1, loss, gx, gp, ws, lw, None) == \
        E.NT_ERR_INVALID
    # mean and broadcast adjoints
    gm, G, ga, gb = (FAKE + 0x1000000 + 0x100000 * k for k in range(4))
    assert lib.nt_pair_reduce_backward(P, gm, None, gm + 16, 16, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_reduce_backward(P, gm, None, None, 16, None) == E.NT_ERR_NULL
    assert lib.nt_pair_reduce_backward(P, gm, G + 16, G, 16, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_broadcast_backward(P, G, G + 64, gb, 16, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_broadcast_backward(P, G, ga, ga + 16, 16, None) == E.NT_ERR_INVALID
    assert lib.nt_pair_broadcast_backward(P, G, ga + 4, gb, 16, None) == E.NT_ERR_ALIGN
    # transition backward
    z, W1, W2, gz, d1, d2 = (FAKE + 0x2000000 + 0x100000 * k for k in range(6))
    tw = FAKE + 0x3000000
    assert lib.nt_transition_backward_workspace_bytes(P, 16, 32, 1, ctypes.byref(need)) == 0
    assert need.value >= 2 * 13 * 32 * 2
    tb = lib.nt_pair_transition_backward
    assert tb(P, z, G, W1, W2, gz, d1, d2, 16, 32, 1, tw, need.value - 1, None) == \
        E.NT_ERR_WORKSPACE
    assert tb(P, z, G, W1, W2, gz, None, d2, 16, 32, 1, tw, need.value, None) == E.NT_ERR_NULL
    assert tb(P, z, G, W1, W2, W1 + 16, d1, d2, 16, 32, 1, tw, need.value, None) == \
        E.NT_ERR_INVALID                                                   # g_z overlaps W1
    assert tb(P, z, G, W1, W2, G + 16, d1, d2, 16, 32, 1, tw, need.value, None) == \
        E.NT_ERR_INVALID                                                   # partial overlap
    assert tb(P, z, G, W1, W2, gz, d1, d2, 16, 36, 1, tw, need.value, None) == E.NT_ERR_INVALID
    assert tb(P, z, G, W1, W2, gz, d1, d2, 16, 32, 5, tw, need.value, None) == E.NT_ERR_DTYPE
    # block backward
    w = _native.NtBlockWeights(*(FAKE + 0x4000000 + 0x10000 * k for k in range(5)))
    g = _native.NtBlockGrads(*(FAKE + 0x5000000 + 0x10000 * k for k in range(5)))
    s, zo, gso, gsi = (FAKE + 0x6000000 + 0x100000 * k for k in range(4))
    bw = FAKE + 0x7000000
    assert lib.nt_block_backward_workspace_bytes(P, 16, 16, 32, 1, ctypes.byref(need)) == 0
    bb = lib.nt_pair_block_backward
    W, Gr = ctypes.byref(w), ctypes.byref(g)
    assert bb(P, s, zo, W, gso, None, gsi, Gr, 16, 16, 32, 1, bw, need.value - 1, None) == \
        E.NT_ERR_WORKSPACE
    assert bb(P, s, zo, W, gso, None, gsi, None, 16, 16, 32, 1, bw, need.value, None) == \
        E.NT_ERR_NULL
    assert bb(P, s, zo, W, gso, None, s, Gr, 16, 16, 32, 1, bw, need.value, None) == \
        E.NT_ERR_INVALID                                                   # g_s_in overlaps s_in
    rect = fake_partition()
    rect.col_offsets = FAKE + 0x9000
    assert bb(ctypes.byref(rect), s, zo, W, gso, None, gsi, Gr, 16, 16, 32, 1, bw, need.value,
              None) == E.NT_ERR_INVALID
    g.W1 = None
    assert bb(P, s, zo, W, gso, None, gsi, Gr, 16, 16, 32, 1, bw, need.value, None) == \
        E.NT_ERR_NULL


def test_non_leading_calls_validate(lib):
    p = fake_partition()
    P = ctypes.byref(p)
    E = _native
    w = _native.NtBlockWeights(*(FAKE + 0x4000000 + 0x10000 * k for k in range(5)))
    W = ctypes.byref(w)
    s, so, z, ws = (FAKE + 0x6000000 + 0x100000 * k for k in range(4))
    need = ctypes.c_size_t()
    assert lib.nt_block_nl_workspace_bytes(P, 3, 16, 16, 32, 1, ctypes.byref(need)) == 0
    assert need.value >= 3 * 5 * 16 * 4 * 3   # a, b, m over T * S rows
    one = ctypes.c_size_t()
    assert lib.nt_block_workspace_bytes(P, 16, 16, 32, 1, ctypes.byref(one)) == 0
    assert need.value > one.value
    bl = lib.nt_pair_block_nl
    assert bl(P, s, so, z, W, 0, 16, 16, 32, 1, ws, need.value, None) == E.NT_ERR_INVALID
    assert bl(P, s, so, z, W, 65, 16, 16, 32, 1, ws, need.value, None) == E.NT_ERR_INVALID
    assert bl(P, s, so, z, W, 5, 16, 128, 32, 1, ws, need.value, None) == E.NT_ERR_INVALID
    assert bl(P, s, so, z, W, 3, 16, 16, 32, 1, ws, need.value - 1, None) == E.NT_ERR_WORKSPACE
    rect = fake_partition()
    rect.col_offsets = FAKE + 0x9000
    assert bl(ctypes.byref(rect), s, so, z, W, 3, 16, 16, 32, 1, ws, need.value, None) == \
        E.NT_ERR_INVALID
    g = _native.NtBlockGrads(*(FAKE + 0x5000000 + 0x10000 * k for k in range(5)))
    assert lib.nt_block_backward_nl_workspace_bytes(P, 3, 16, 16, 32, 1, ctypes.byref(need)) == 0
    bb = lib.nt_pair_block_backward_nl
    gso, gsi = FAKE + 0x7000000, FAKE + 0x7100000
    assert bb(P, s, z, W, gso, None, gsi, ctypes.byref(g), 3, 16, 16, 32, 1, ws,
              need.value - 1, None) == E.NT_ERR_WORKSPACE
    assert bb(P, s, z, W, gso, None, gsi, ctypes.byref(g), 9, 16, 64, 32, 1, ws,
              need.value, None) == E.NT_ERR_INVALID


def test_chain_validates(lib):
    """nt_pair_chain rejects bad arguments before anything is launched."""
    p = fake_partition()
    P = ctypes.byref(p)
    s, so, z = FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000
    w = (_native.NtBlockWeights * 2)(
        _native.NtBlockWeights(*(FAKE + 0x400000 + 0x1000 * k for k in range(5))),
        _native.NtBlockWeights(*(FAKE + 0x500000 + 0x1000 * k for k in range(5))))
    ws = FAKE + 0x800000
    E = _native
    one, two = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.nt_chain_workspace_bytes(P, 1, 16, 16, 32, 1, ctypes.byref(one)) == 0
    assert lib.nt_chain_workspace_bytes(P, 2, 16, 16, 32, 1, ctypes.byref(two)) == 0
    blk = ctypes.c_size_t()
    assert lib.nt_block_workspace_bytes(P, 16, 16, 32, 1, ctypes.byref(blk)) == 0
    assert one.value == blk.value                    # one block: the block's workspace
    assert two.value >= blk.value + 5 * 16 * 2       # plus a [T, c_s] bf16 buffer
    assert lib.nt_chain_workspace_bytes(P, 0, 16, 16, 32, 1, ctypes.byref(one)) == \
        E.NT_ERR_INVALID
    need = two.value
    ch = lib.nt_pair_chain
    assert ch(P, s, so, z, w, 0, 16, 16, 32, 1, ws, need, None) == E.NT_ERR_INVALID
    assert ch(P, s, so, z, None, 2, 16, 16, 32, 1, ws, need, None) == E.NT_ERR_NULL
    assert ch(P, s, so, z, w, 2, 16, 16, 32, 7, ws, need, None) == E.NT_ERR_DTYPE
    assert ch(P, s, so, z, w, 2, 16, 16, 32, 1, ws, need - 1, None) == E.NT_ERR_WORKSPACE
    assert ch(P, s, so, z, w, 2, 16, 16, 32, 1, None, need, None) == E.NT_ERR_NULL
    assert ch(P, None, so, z, w, 2, 16, 16, 32, 1, ws, need, None) == E.NT_ERR_NULL
    assert ch(P, s, s + 32, z, w, 2, 16, 16, 32, 1, ws, need, None) == E.NT_ERR_INVALID
    assert ch(P, s, so, so + 32, w, 2, 16, 16, 32, 1, ws, need, None) == E.NT_ERR_INVALID
    assert ch(P, s, so, z, w, 2, 16, 16, 32, 1, z + 64, need, None) == E.NT_ERR_INVALID
    bad = (_native.NtBlockWeights * 2)(w[0], _native.NtBlockWeights(
        FAKE + 0x500000, None, FAKE + 0x502000, FAKE + 0x503000, FAKE + 0x504000))
    assert ch(P, s, so, z, bad, 2, 16, 16, 32, 1, ws, need, None) == E.NT_ERR_NULL
    wz = (_native.NtBlockWeights * 2)(w[0], _native.NtBlockWeights(
        z, FAKE + 0x501000, FAKE + 0x502000, FAKE + 0x503000, FAKE + 0x504000))
    assert ch(P, s, so, z, wz, 2, 16, 16, 32, 1, ws, need, None) == E.NT_ERR_INVALID
    rect = fake_partition()
    rect.col_offsets = FAKE + 0x9000
    assert ch(ctypes.byref(rect), s, so, z, w, 2, 16, 16, 32, 1, ws, need, None) == \
        E.NT_ERR_INVALID


# ------------------------------------------------ binding extent checks (host)
def _binding_partition(B=2, T=5, cells=13):
    """A Partition whose buffer lives on the CPU: every tensor below is a CPU
    tensor too, and each call is rejected by the binding's shape, dtype,
    device or workspace checks before any native launch."""
    torch = pytest.importorskip("torch")
    import padding_free_pair_amd as nt
    return nt, torch, nt.Partition(fake_partition(B, T, cells), torch.empty(256, dtype=torch.uint8),
                                   np.array([2, 3], dtype=np.int32))


def _block_args(torch, T=5, cells=13, c_s=16, c_z=8, hidden=16, dt=None):
    dt = dt or torch.float32
    s = torch.zeros((T, c_s), dtype=dt)
    w = {"Wa": torch.zeros((c_z, c_s), dtype=dt), "Wb": torch.zeros((c_z, c_s), dtype=dt),
         "W1": torch.zeros((hidden, c_z), dtype=dt), "W2": torch.zeros((c_z, hidden), dtype=dt),
         "Wo": torch.zeros((c_s, c_z), dtype=dt)}
    return s, w


@pytest.mark.parametrize("case", ["s_rows", "s_out", "z_out", "W1", "Wo", "workspace",
                                  "chain_block1", "device"])
def test_binding_rejects_bad_extents(lib, case):
    nt, torch, p = _binding_partition()
    s, w = _block_args(torch)
    kw = {}
    if case == "s_rows":
        s = torch.zeros((4, 16))
    elif case == "s_out":
        kw["s_out"] = torch.zeros((5, 8))
    elif case == "z_out":
        kw["z_out"] = torch.zeros((12, 8))
    elif case == "W1":
        w["W1"] = torch.zeros((16, 16))
    elif case == "Wo":
        w["Wo"] = torch.zeros((8, 16))
    elif case == "workspace":
        kw["workspace"] = torch.zeros(8, dtype=torch.uint8)
    elif case == "device":
        kw["workspace"] = torch.zeros(1 << 16, dtype=torch.uint8, device="meta")
    if case == "chain_block1":
        w2 = dict(w)
        w2["W2"] = torch.zeros((8, 24))
        with pytest.raises(ValueError, match="block 1 W2"):
            nt.nt_pair_chain(p, s, [w, w2])
        return
    with pytest.raises(ValueError):
        nt.nt_pair_block(p, s, w, **kw)


def test_binding_rejects_bad_stage_extents(lib):
    nt, torch, p = _binding_partition()
    a = torch.zeros((5, 8))
    with pytest.raises(ValueError, match="b has shape"):
        nt.nt_pair_broadcast(p, a, torch.zeros((4, 8)))
    with pytest.raises(ValueError, match="z_in has shape"):
        nt.nt_pair_transition(p, torch.zeros((14, 8)), torch.zeros((16, 8)), torch.zeros((8, 16)))
    with pytest.raises(ValueError, match="W2 has shape"):
        nt.nt_pair_broadcast_transition(p, a, a, torch.zeros((16, 8)), torch.zeros((16, 8)))
    with pytest.raises(ValueError, match="m has shape"):
        nt.nt_pair_reduce(p, torch.zeros((13, 8)), m=torch.zeros((13, 8)))
    with pytest.raises(ValueError, match="g_z has shape"):
        nt.nt_pair_broadcast_backward(p, torch.zeros((12, 8)))
    with pytest.raises(ValueError, match="dW1 has shape"):
        nt.nt_pair_transition_backward(p, torch.zeros((13, 8)), torch.zeros((13, 8)),
                                       torch.zeros((16, 8)), torch.zeros((8, 16)),
                                       dW1=torch.zeros((8, 16)))
    s, w = _block_args(torch)
    with pytest.raises(ValueError, match="dWa has shape"):
        grads = {k: torch.zeros(v.shape) for k, v in w.items()}
        grads["Wa"] = torch.zeros((16, 8))
        nt.nt_pair_block_backward(p, s, torch.zeros((13, 8)), w, torch.zeros((5, 16)),
                                  grads=grads)


def test_noalloc_rejects_oversized_partition(lib):
    """The static scratch holds 16 MiB: a partition needing more is refused
    with NT_ERR_WORKSPACE before any device work (T = 10,923 at c_z = 128)."""
    p = fake_partition(B=1, T=10923, cells=10923 * 10923)
    w = _native.NtBlockWeights(FAKE + 0x400000, FAKE + 0x410000, FAKE + 0x420000,
                               FAKE + 0x430000, FAKE + 0x440000)
    st = lib.nt_pair_block_noalloc(ctypes.byref(p), FAKE + 0x100000, FAKE + 0x200000,
                                   FAKE + 0x300000, ctypes.byref(w), 384, 128, 512,
                                   _native.NT_BF16, None)
    assert st == _native.NT_ERR_WORKSPACE
    assert "static scratch" in lib.nt_last_error().decode()


def test_block_params_layout_and_validation(lib):
    """nt_block_params: int32 kind, float ln_eps, ten pointers. The transition
    kind is checked before anything is enqueued: an unknown kind, the SwiGLU
    kind in fp32, widths it does not take, a negative epsilon."""
    assert ctypes.sizeof(_native.NtBlockParams) == 8 + 10 * 8
    assert _native.NtBlockParams.Wa.offset == 8
    assert ctypes.sizeof(_native.NtBlockParamGrads) == 10 * 8
    p = fake_partition()
    s, so, z = FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000
    ws = FAKE + 0x800000

    def call(kind, dtype=_native.NT_BF16, c_z=128, hidden=512, eps=1e-5):
        w = _native.NtBlockParams()
        w.kind, w.ln_eps = kind, eps
        for k, name in enumerate(_native.PARAM_NAMES):
            setattr(w, name, FAKE + 0x400000 + 0x40000 * k)
        return lib.nt_pair_block_ex(ctypes.byref(p), s, None, so, z, ctypes.byref(w), 64, c_z,
                                    hidden, dtype, ws, 1 << 30, None)

    assert call(7) == _native.NT_ERR_INVALID
    assert "transition kind" in lib.nt_last_error().decode()
    assert call(_native.NT_TRANSITION_LN_SWIGLU, dtype=_native.NT_F32) == _native.NT_ERR_DTYPE
    assert call(_native.NT_TRANSITION_LN_SWIGLU, c_z=96) == _native.NT_ERR_INVALID
    assert call(_native.NT_TRANSITION_LN_SWIGLU, hidden=520) == _native.NT_ERR_INVALID
    assert call(_native.NT_TRANSITION_LN_SWIGLU, eps=-1.0) == _native.NT_ERR_INVALID
    need = ctypes.c_size_t()
    assert lib.nt_block_backward_ex_workspace_bytes(ctypes.byref(p), 9, 64, 128, 512,
                                                    _native.NT_BF16,
                                                    ctypes.byref(need)) == _native.NT_ERR_INVALID
    assert lib.nt_block_backward_ex_workspace_bytes(ctypes.byref(p),
                                                    _native.NT_TRANSITION_LN_SWIGLU, 64, 128, 512,
                                                    _native.NT_BF16, ctypes.byref(need)) == 0
    assert need.value > 0
