"""Plain float64 implementation of the packed single-pair-single block.

TEST INFRASTRUCTURE (see the package docstring): callers are tests/, the
smoke check and the CPU-baseline leg of the benchmark only.

Notation follows the DanLing NestedTensor paper (arXiv 2609.30379):
N_i sample lengths, eta_i single offsets, o_i pair (sample) offsets,
row splits the second-level partition of Figure 2. Arrays are numpy float64;
``w`` is a dict with Wa, Wb [c_z, c_s], W1 [hidden, c_z], W2 [c_z, hidden],
Wo [c_s, c_z] stored [out, in] (Section 3.3's V W^T).
"""
from __future__ import annotations

import numpy as np

_CHUNK_ROWS = 1 << 16   # bound the hidden activations' memory in transition()


# ------------------------------------------------------------------ structure
def partition(lengths):
    """Offsets and row splits of a square pair partition.

    Section 3.1 Eq. 2 with p_i = N_i (singles) and p_i = N_i^2 (pairs);
    Appendix A: o_0 = 0, o_{i+1} - o_i = p_i. The second-level row splits
    (Figure 2) start pair row r of sample i at Eq. 3's o_i + r * N_i and
    close with the total cell count.
    """
    N = [int(n) for n in lengths]
    eta, o = [0], [0]
    for n in N:
        eta.append(eta[-1] + n)
        o.append(o[-1] + n * n)
    row_splits, row_sample = [], []
    for i, n in enumerate(N):
        for r in range(n):
            row_splits.append(o[i] + r * n)
            row_sample.append(i)
    row_splits.append(o[-1])
    return {
        "B": len(N), "T": eta[-1], "cells": o[-1], "n_max": max(N, default=0),
        "single_offsets": np.array(eta, dtype=np.int64),
        "pair_offsets": np.array(o, dtype=np.int64),
        "row_splits": np.array(row_splits, dtype=np.int64),
        "row_sample": np.array(row_sample, dtype=np.int32),
    }


def decode_cells(lengths):
    """(sample, row, col) of every packed cell, by enumerating Eq. 3.

    Cell o_i + a * N_i + b belongs to sample i, row a, column b.
    """
    p = partition(lengths)
    cells = p["cells"]
    sample = np.full(cells, -1, dtype=np.int64)
    row = np.full(cells, -1, dtype=np.int64)
    col = np.full(cells, -1, dtype=np.int64)
    for i, n in enumerate(int(x) for x in lengths):
        if n == 0:
            continue
        a = np.repeat(np.arange(n), n)
        b = np.tile(np.arange(n), n)
        ell = p["pair_offsets"][i] + a * n + b
        sample[ell] = i
        row[ell] = a
        col[ell] = b
    return sample, row, col


# ------------------------------------------------------ rectangular pairs
# Section 3.1 packs rectangular pairs (N_i, M_i, C) as (sum N_i M_i, C); the
# row axis follows one single partition (N_i, offsets eta), the column axis a
# second one (M_i, offsets mu). Appendix A.1's rectangular variant builds the
# pair from distinct row and column inputs and divides its column mean by M_i
# (Eq. 4 groups the M_i cells of a row). With M = N every function below is
# the square one.
def partition_rect(rows, cols):
    """Offsets and row splits of a rectangular pair partition: eta over the
    row lengths N_i, mu over the column lengths M_i, o over N_i M_i (Eq. 2),
    and pair row r of sample i starting at o_i + r M_i (Eq. 3)."""
    N = [int(n) for n in rows]
    M = [int(m) for m in cols]
    if len(N) != len(M):
        raise ValueError("row and column length vectors differ in size")
    eta, mu, o = [0], [0], [0]
    for n, m in zip(N, M):
        eta.append(eta[-1] + n)
        mu.append(mu[-1] + m)
        o.append(o[-1] + n * m)
    row_splits, row_sample = [], []
    for i, (n, m) in enumerate(zip(N, M)):
        for r in range(n):
            row_splits.append(o[i] + r * m)
            row_sample.append(i)
    row_splits.append(o[-1])
    return {
        "B": len(N), "T": eta[-1], "T_cols": mu[-1], "cells": o[-1],
        "single_offsets": np.array(eta, dtype=np.int64),
        "col_offsets": np.array(mu, dtype=np.int64),
        "pair_offsets": np.array(o, dtype=np.int64),
        "row_splits": np.array(row_splits, dtype=np.int64),
        "row_sample": np.array(row_sample, dtype=np.int32),
    }


def decode_cells_rect(rows, cols):
    """(sample, row, col) of every packed cell: cell o_i + a M_i + b belongs to
    sample i, row a < N_i, column b < M_i."""
    p = partition_rect(rows, cols)
    sample = np.full(p["cells"], -1, dtype=np.int64)
    row = np.full(p["cells"], -1, dtype=np.int64)
    col = np.full(p["cells"], -1, dtype=np.int64)
    for i, (n, m) in enumerate(zip(rows, cols)):
        n, m = int(n), int(m)
        if n * m == 0:
            continue
        a = np.repeat(np.arange(n), m)
        b = np.tile(np.arange(m), n)
        ell = p["pair_offsets"][i] + a * m + b
        sample[ell], row[ell], col[ell] = i, a, b
    return sample, row, col


def broadcast_rect(rows, cols, a, b):
    """z[o_i + r M_i + c] = a[eta_i + r] + b[mu_i + c]: a [sum N_i, C] are the
    row singles' projections, b [sum M_i, C] the column singles'."""
    p = partition_rect(rows, cols)
    sample, row, col = decode_cells_rect(rows, cols)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return a[p["single_offsets"][sample] + row] + b[p["col_offsets"][sample] + col]


def reduce_mean_rect(rows, cols, zt):
    """Eq. 4's column sum over the M_i cells of each pair row, divided by M_i.
    Returns [sum N_i, C] in the row singles' partition; a row of a sample with
    M_i = 0 has no cells and no mean (NaN)."""
    zt = np.asarray(zt, dtype=np.float64)
    out = []
    o = 0
    for n, m in zip((int(x) for x in rows), (int(x) for x in cols)):
        if n == 0:
            continue
        if m == 0:
            out.append(np.full((n, zt.shape[1]), np.nan))
            continue
        out.append(zt[o:o + n * m].reshape(n, m, zt.shape[1]).sum(axis=1) / m)
        o += n * m
    return np.concatenate(out) if out else np.zeros((0, zt.shape[1]))


def block_rect(rows, cols, s_rows, s_cols, w):
    """The rectangular single-pair-single block (Appendix A.1's rectangular
    variant): pair rows from s_rows [sum N_i, c_s], columns from s_cols
    [sum M_i, c_s]; returns (s_rows + m Wo^T, z~)."""
    a = project(s_rows, w["Wa"])
    b = project(s_cols, w["Wb"])
    zt = transition(broadcast_rect(rows, cols, a, b), w["W1"], w["W2"])
    m = reduce_mean_rect(rows, cols, zt)
    return np.asarray(s_rows, dtype=np.float64) + project(m, w["Wo"]), zt


# ------------------------------------------------------------------ stages
def project(x, W):
    """Dense projection on packed rows: x W^T (Section 3.3, no bias)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def broadcast(lengths, a, b):
    """Pair state of Eq. 1's first line: z_i[r, c] = a_i[r] + b_i[c].

    Per sample the row operand a (left, unsqueeze(-2) in Figure 3) and the
    column operand b (right, unsqueeze(-3)) form an N_i x N_i x C block; its
    rows are packed row-major at o_i (Eq. 2/3). No activation (Appendix A.1).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    blocks = []
    eta = 0
    for n in (int(x) for x in lengths):
        A = a[eta:eta + n]
        Bm = b[eta:eta + n]
        blocks.append((A[:, None, :] + Bm[None, :, :]).reshape(n * n, a.shape[1]))
        eta += n
    if not blocks:
        return np.zeros((0, a.shape[1]))
    return np.concatenate(blocks, axis=0)


def transition(z, W1, W2):
    """Residual cell-local transition z + relu(z W1^T) W2^T (Eq. 1's second line
    with the ReLU MLP as the feature update)."""
    z = np.asarray(z, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    out = np.empty_like(z)
    for s in range(0, z.shape[0], _CHUNK_ROWS):
        zc = z[s:s + _CHUNK_ROWS]
        h = np.maximum(zc @ W1.T, 0.0)
        out[s:s + _CHUNK_ROWS] = zc + h @ W2.T
    return out


def layer_norm(z, gamma, beta, eps):
    """LN over the pair features of every cell (the LN_{C_p} of Eq. 1's second
    line): (z - mean) / sqrt(var + eps) * gamma + beta, with the mean and the
    biased variance taken over the c_z features of the cell."""
    z = np.asarray(z, dtype=np.float64)
    mu = z.mean(axis=-1, keepdims=True)
    var = np.square(z - mu).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + eps) * np.asarray(gamma, dtype=np.float64) \
        + np.asarray(beta, dtype=np.float64)


def transition_swiglu(z, gamma, beta, Wg, Wu, Wd, eps=1e-5):
    """The paper's measured transition (Eq. 1's second line; Appendix A.1: a
    residual, pre-normalised SwiGLU update of expansion four): with x = LN(z),
    z + (silu(x Wg^T) * (x Wu^T)) Wd^T, silu(g) = g / (1 + exp(-g)).
    Wg, Wu are [hidden, c_z] and Wd is [c_z, hidden] ([out, in])."""
    z = np.asarray(z, dtype=np.float64)
    Wg, Wu, Wd = (np.asarray(w, dtype=np.float64) for w in (Wg, Wu, Wd))
    out = np.empty_like(z)
    for s in range(0, z.shape[0], _CHUNK_ROWS):
        zc = z[s:s + _CHUNK_ROWS]
        x = layer_norm(zc, gamma, beta, eps)
        g = x @ Wg.T
        u = x @ Wu.T
        out[s:s + _CHUNK_ROWS] = zc + (g / (1.0 + np.exp(-g)) * u) @ Wd.T
    return out


def reduce_mean(lengths, zt):
    """Column mean of Eq. 1's third line: Eq. 4's grouped sum over the column
    index b, then division by N_i. Returns [T, C] with the singles' partition."""
    zt = np.asarray(zt, dtype=np.float64)
    out = []
    o = 0
    for n in (int(x) for x in lengths):
        if n == 0:
            continue
        blk = zt[o:o + n * n].reshape(n, n, zt.shape[1])
        out.append(blk.sum(axis=1) / n)
        o += n * n
    if not out:
        return np.zeros((0, zt.shape[1]))
    return np.concatenate(out, axis=0)


def block(lengths, s, w):
    """One single-pair-single block (Eq. 1, Figure 3). Returns (s_out, z_out)."""
    s = np.asarray(s, dtype=np.float64)
    a = project(s, w["Wa"])
    b = project(s, w["Wb"])
    z = broadcast(lengths, a, b)
    zt = transition(z, w["W1"], w["W2"])
    m = reduce_mean(lengths, zt)
    return s + project(m, w["Wo"]), zt


def chain(lengths, s, ws):
    """Blocks applied in sequence: each block's singles feed the next, the pair
    state is rebuilt from them. Returns the final singles and last pair state."""
    z = None
    for w in ws:
        s, z = block(lengths, s, w)
    return s, z


def block_swiglu(lengths, s, w, eps=1e-5):
    """The block with the paper's own transition (Eq. 1 with h o LN_{C_p};
    Appendix A.1: a residual, pre-normalised SwiGLU of expansion four) in
    place of the ReLU MLP; every other step as in block(). w holds Wa, Wb,
    Wo and the transition's ln_gamma, ln_beta, Wg, Wu, Wd. Returns
    (s_out, z_out)."""
    s = np.asarray(s, dtype=np.float64)
    a = project(s, w["Wa"])
    b = project(s, w["Wb"])
    z = broadcast(lengths, a, b)
    zt = transition_swiglu(z, w["ln_gamma"], w["ln_beta"], w["Wg"], w["Wu"], w["Wd"], eps)
    m = reduce_mean(lengths, zt)
    return s + project(m, w["Wo"]), zt


def chain_swiglu(lengths, s, ws, eps=1e-5):
    """SwiGLU blocks in sequence, as chain() chains ReLU blocks."""
    z = None
    for w in ws:
        s, z = block_swiglu(lengths, s, w, eps)
    return s, z


# ------------------------------------------------- independent forms (pins)
def dense_block(X, w):
    """The dense per-sample computation of one sample X [N, c_s] (Appendix A's
    reference semantics). Returns (X_out [N, c_s], P_out [N, N, c_z])."""
    X = np.asarray(X, dtype=np.float64)
    U = X @ w["Wa"].T
    V = X @ w["Wb"].T
    P = U[:, None, :] + V[None, :, :]
    H = np.maximum(np.einsum("rcf,hf->rch", P, w["W1"]), 0.0)
    Pt = P + np.einsum("rch,fh->rcf", H, w["W2"])
    n = X.shape[0]
    M = Pt.sum(axis=1) / n
    return X + M @ w["Wo"].T, Pt


def block_padded_masked(lengths, s, w):
    """The same block over a B x N_max x N_max envelope: zero-padded singles,
    a validity mask (true = valid, Appendix A) and a mean over valid columns.
    Valid rows and cells are then packed."""
    N = np.asarray(lengths, dtype=np.int64)
    B = N.size
    nmax = int(N.max(initial=0))
    s = np.asarray(s, dtype=np.float64)
    cs = s.shape[1]
    S = np.zeros((B, nmax, cs))
    valid = np.zeros((B, nmax), dtype=bool)
    eta = 0
    for i, n in enumerate(N):
        S[i, :n] = s[eta:eta + n]
        valid[i, :n] = True
        eta += n
    U = S @ w["Wa"].T
    V = S @ w["Wb"].T
    P = U[:, :, None, :] + V[:, None, :, :]
    H = np.maximum(P @ w["W1"].T, 0.0)
    Pt = P + H @ w["W2"].T
    colmask = valid[:, None, :, None].astype(np.float64)
    cnt = np.maximum(N, 1).astype(np.float64)[:, None, None]
    M = (Pt * colmask).sum(axis=2) / cnt
    So = S + M @ w["Wo"].T
    s_out = np.concatenate([So[i, :n] for i, n in enumerate(N)] or [np.zeros((0, cs))])
    z_out = np.concatenate([Pt[i, :n, :n].reshape(n * n, Pt.shape[-1]) for i, n in enumerate(N)]
                           or [np.zeros((0, Pt.shape[-1]))])
    return s_out, z_out


def block_gather(lengths, s, w):
    """The explicit-packed form of Figure 3's last line: caller-built row and
    column gather indices, a segmented sum (np.add.reduceat) over row splits."""
    N = np.asarray(lengths, dtype=np.int64)
    s = np.asarray(s, dtype=np.float64)
    rows, cols, starts, counts = [], [], [], []
    eta = 0
    o = 0
    for n in N:
        n = int(n)
        r = np.repeat(np.arange(n), n)
        c = np.tile(np.arange(n), n)
        rows.append(eta + r)
        cols.append(eta + c)
        starts.extend(o + np.arange(n) * n)
        counts.extend([n] * n)
        eta += n
        o += n * n
    rows = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    cols = np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)
    a = s @ w["Wa"].T
    b = s @ w["Wb"].T
    z = a[rows] + b[cols]
    zt = z + np.maximum(z @ w["W1"].T, 0.0) @ w["W2"].T
    if len(starts):
        m = np.add.reduceat(zt, np.asarray(starts), axis=0) / np.asarray(counts, dtype=np.float64)[:, None]
    else:
        m = np.zeros((0, zt.shape[1]))
    return s + m @ w["Wo"].T, zt


def block_bruteforce(lengths, s, w):
    """Scalar loops over (sample, row, column, feature): tiny inputs only."""
    s = [list(map(float, row)) for row in np.asarray(s, dtype=np.float64)]
    Wa, Wb, W1, W2, Wo = (np.asarray(w[k], dtype=np.float64).tolist()
                          for k in ("Wa", "Wb", "W1", "W2", "Wo"))
    cz, cs, hd = len(Wa), len(Wa[0]), len(W1)

    def lin(x, W):
        return [sum(W[o][k] * x[k] for k in range(len(x))) for o in range(len(W))]

    s_out = [row[:] for row in s]
    z_out = []
    eta = 0
    for n in (int(x) for x in lengths):
        for r in range(n):
            acc = [0.0] * cz
            for c in range(n):
                ar = lin(s[eta + r], Wa)
                bc = lin(s[eta + c], Wb)
                z = [ar[f] + bc[f] for f in range(cz)]
                h = [max(v, 0.0) for v in lin(z, W1)]
                y = lin(h, W2)
                zt = [z[f] + y[f] for f in range(cz)]
                z_out.append(zt)
                for f in range(cz):
                    acc[f] += zt[f]
            m = [acc[f] / n for f in range(cz)]
            g = lin(m, Wo)
            for k in range(cs):
                s_out[eta + r][k] = s[eta + r][k] + g[k]
        eta += n
    del hd
    return np.array(s_out, dtype=np.float64).reshape(-1, cs), \
        np.array(z_out, dtype=np.float64).reshape(-1, cz)


# ---------------------------------------------- sampled evaluation (large)
def broadcast_cells(lengths, a, b, cell_ids):
    """broadcast() at selected packed cells only: a[eta_i + r] + b[eta_i + c]."""
    p = partition(lengths)
    sample, row, col = _decode_some(p, lengths, np.asarray(cell_ids, dtype=np.int64))
    eta = p["single_offsets"][sample]
    return np.asarray(a, dtype=np.float64)[eta + row] + np.asarray(b, dtype=np.float64)[eta + col]


def block_cells(lengths, s, w, cell_ids):
    """z_out of one block at selected packed cells only (the transition is
    cell-local, so each cell needs just its row and column singles)."""
    p = partition(lengths)
    sample, row, col = _decode_some(p, lengths, np.asarray(cell_ids, dtype=np.int64))
    eta = p["single_offsets"][sample]
    s = np.asarray(s, dtype=np.float64)
    z = project(s[eta + row], w["Wa"]) + project(s[eta + col], w["Wb"])
    return transition(z, w["W1"], w["W2"])


def block_rows(lengths, s, w, row_ids):
    """(m, s_out) of one block at selected single rows only; each row needs
    its whole pair row (N_i cells)."""
    p = partition(lengths)
    s = np.asarray(s, dtype=np.float64)
    row_ids = np.asarray(row_ids, dtype=np.int64)
    ms, so = [], []
    for g in row_ids:
        i = int(p["row_sample"][g])
        n = int(lengths[i])
        eta = int(p["single_offsets"][i])
        a = project(s[g:g + 1], w["Wa"])
        b = project(s[eta:eta + n], w["Wb"])
        zt = transition(a + b, w["W1"], w["W2"])
        m = zt.sum(axis=0, keepdims=True) / n
        ms.append(m[0])
        so.append((s[g:g + 1] + project(m, w["Wo"]))[0])
    return np.array(ms).reshape(len(row_ids), -1), np.array(so).reshape(len(row_ids), -1)


def _decode_some(p, lengths, t):
    """Eq. 3 inverted: the sample whose offset range holds t, then row-major
    (row, col) inside its N_i x N_i block."""
    o = p["pair_offsets"]
    n = np.asarray(lengths, dtype=np.int64)
    sample = np.searchsorted(o, t, side="right") - 1
    local = t - o[sample]
    row = local // n[sample]
    col = local - row * n[sample]
    return sample, row, col


# ------------------------------------------------------------- bf16 rounding
def bf16_bits(x):
    """Round float64 values to bfloat16 (nearest, ties to even) in one step.

    bfloat16 keeps 8 significand bits, so the 45 low fraction bits of the
    float64 are rounded away; the result is then an exact float32 whose high
    16 bits are the bfloat16 pattern. Finite, normal-range inputs.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    drop = np.uint64(45)
    lsb = (u >> drop) & np.uint64(1)
    u = (u + (np.uint64(1) << (drop - np.uint64(1))) - np.uint64(1) + lsb) >> drop << drop
    r32 = u.view(np.float64).astype(np.float32)
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_bf16(x):
    """float64 value of bf16_bits(x)."""
    bits = bf16_bits(x)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
