"""ReLU decisions that the rounding of the transition's operand may move.

The gradient of z' = z + relu(z W1^T) W2^T holds the mask [z W1^T > 0]. The
oracle takes it on the exact float64 pair state; a kernel takes it on the
pre-activation it computes from its stored operand (z rounded to bf16 for
bf16 storage, or fp32 z built from fp32 projections) with an fp32 sum. Where
the exact pre-activation lies within that error of zero, the two decisions
may differ, and the gradient then moves by one hidden unit's whole term: a
jump, not a rounding error, which no relative tolerance covers.

The tests therefore:
  1. bound, from the oracle's exact values only, the interval the kernel's
     pre-activation of every (cell, unit) pair lies in, and list the pairs
     whose decision can differ from the exact one (`candidates`);
  2. choose, for each group of candidates one observable output row depends
     on (a cell's g_z, or a unit's row of dW1), the subset of flips that best
     explains the kernel's output (`fit_flips`, exhaustive over the subsets);
  3. add the exact effect of those flips to the oracle's gradients (every
     step after the mask is linear in g_H) and compare EVERY output element
     with the tolerance, with no cell left out.
A kernel error that is not a flip of a listed pair cannot be explained this
way and fails step 3. The reference values stay the plain oracle's.
"""
import itertools

import numpy as np

import oracle

U32 = 2.0 ** -24  # fp32 unit roundoff


def gamma(n):
    """gamma_n = n u / (1 - n u): the relative error bound of an n-term fp32
    sum of exact products, whatever the summation order."""
    return n * U32 / (1.0 - n * U32)


def operand_interval(z_exact, e_z, bf16: bool):
    """The kernel's operand is z_exact perturbed by at most e_z (fp32 work
    before it), then rounded once to bf16 if `bf16`. Returns (zq, dz): every
    element of the kernel's operand lies in [zq - dz, zq + dz]. Rounding is
    monotone, so the extremes come from the interval's ends."""
    if not bf16:
        return z_exact, e_z
    zq = oracle.round_bf16(z_exact)
    lo = oracle.round_bf16(z_exact - e_z)
    hi = oracle.round_bf16(z_exact + e_z)
    return zq, np.maximum(np.abs(hi - zq), np.abs(zq - lo))


def candidates(z_exact, W1, zq, dz, chunk=1 << 16):
    """The (cell, unit) pairs whose relu decision may differ between the
    exact pre-activation z_exact W1^T and the kernel's, which lies within
    dz |W1|^T + gamma_{c_z} (|zq| + dz) |W1|^T of zq W1^T. Returns the cell
    and unit index arrays and the exact pre-activation of each pair."""
    W1a = np.abs(W1).T
    g = gamma(W1.shape[1])
    cells, units, pres = [], [], []
    for s in range(0, z_exact.shape[0], chunk):
        pre = z_exact[s:s + chunk] @ W1.T
        center = zq[s:s + chunk] @ W1.T
        d = dz[s:s + chunk]
        err = d @ W1a + g * ((np.abs(zq[s:s + chunk]) + d) @ W1a)
        c, u = np.nonzero(np.where(pre > 0, center - err <= 0, center + err > 0))
        cells.append(c + s)
        units.append(u)
        pres.append(pre[c, u])
    if not cells:
        return np.zeros(0, int), np.zeros(0, int), np.zeros(0)
    return np.concatenate(cells), np.concatenate(units), np.concatenate(pres)


def unit_terms(G, W2, cells, units):
    """g_P = (G W2)[cell, unit] at the listed pairs."""
    return np.einsum("ij,ji->i", G[cells], W2[:, units]) if len(cells) else np.zeros(0)


def _best_subset(r, V, max_candidates=12):
    """The 0/1 weights x minimising max |r - x V| (V: [k, d]), over all 2^k
    subsets. A group with more candidates than max_candidates is refused:
    the test's batch is then too large for its window."""
    k = V.shape[0]
    if k > max_candidates:
        raise AssertionError(f"{k} candidates in one group: use a smaller batch")
    masks = np.array(list(itertools.product((0.0, 1.0), repeat=k)))  # [2^k, k]
    return masks[int(np.argmin(np.max(np.abs(r[None, :] - masks @ V), axis=1)))]


def fit_flips(resid, group, vectors):
    """resid [n_groups, d]: kernel output minus reference, one row per group;
    group [n]: the group of each candidate; vectors [n, d]: the change a
    flip of that candidate makes to its group's row. For every group, the
    subset of its candidates whose summed vectors leave the smallest
    max-abs residual. Returns a boolean [n]: the flips chosen."""
    chosen = np.zeros(len(group), dtype=bool)
    if len(group) == 0:
        return chosen
    order = np.argsort(group, kind="stable")
    g_sorted = group[order]
    starts = np.flatnonzero(np.r_[True, g_sorted[1:] != g_sorted[:-1]])
    ends = np.r_[starts[1:], len(order)]
    for a, b in zip(starts, ends):
        idx = order[a:b]
        chosen[idx] = _best_subset(resid[g_sorted[a]], vectors[idx]).astype(bool)
    return chosen


def flip_terms(pre, gP):
    """g_H change of each candidate when flipped: a unit the exact mask keeps
    (pre > 0) loses its term g_P, one it drops gains it."""
    return np.where(pre > 0, -1.0, 1.0) * gP


def transition_reference(z, W1, W2, G, got_gz):
    """Oracle gradients of the transition at the stored operand z (both sides
    read the same z), with the flips that best explain the kernel's g_z (one
    group per cell) added. Returns (g_z, dW1, dW2, flips, candidates)."""
    rz, r1, r2 = oracle.transition_backward(z, W1, W2, G)
    cells, units, pre = candidates(z, W1, z, np.zeros_like(z))
    dh = flip_terms(pre, unit_terms(G, W2, cells, units))
    vec = dh[:, None] * W1[units]
    chosen = fit_flips(got_gz - rz, cells, vec)
    np.add.at(rz, cells[chosen], vec[chosen])
    np.add.at(r1, units[chosen], dh[chosen, None] * z[cells[chosen]])
    return rz, r1, r2, int(chosen.sum()), len(cells)


def block_reference(lengths, s, W, g_s_out, g_z_out, got_dW1, bf16, S=1):
    """Oracle gradients of the block (S slices sharing the weights; S = 1 is
    the leading layout), with the flips that best explain the kernel's dW1
    (one group per hidden unit) carried through every later adjoint: g_z,
    the broadcast's row and column sums, the single gradient and dWa, dWb.
    The kernel's operand is bf16(fp32(a + b)) for bf16 (fp32(a + b) for
    fp32), a and b fp32 dot products of c_s exact terms. Returns (reference
    dict, flips, candidates)."""
    s = np.asarray(s, dtype=np.float64)
    T = s.shape[0]
    x = s.reshape(T, S, -1)
    gs = np.asarray(g_s_out, dtype=np.float64).reshape(T, S, -1)
    c_s, c_z = x.shape[2], W["Wa"].shape[0]
    if S == 1:
        ref = oracle.block_backward(lengths, s, W, g_s_out, g_z_out)
    else:
        ref = oracle.block_backward_nl(lengths, s, W, S, g_s_out, g_z_out)
    slices = []
    for k in range(S):
        xk = x[:, k, :]
        zx = oracle.broadcast(lengths, oracle.project(xk, W["Wa"]), oracle.project(xk, W["Wb"]))
        e = oracle.broadcast(lengths, gamma(c_s) * (np.abs(xk) @ np.abs(W["Wa"]).T),
                             gamma(c_s) * (np.abs(xk) @ np.abs(W["Wb"]).T)) + U32 * np.abs(zx)
        zq, dz = operand_interval(zx, e, bf16)
        cells, units, pre = candidates(zx, W["W1"], zq, dz)
        G = oracle.reduce_mean_backward(lengths, lengths, gs[:, k, :] @ W["Wo"])
        if g_z_out is not None:
            G = G + np.asarray(g_z_out, dtype=np.float64)[:, k * c_z:(k + 1) * c_z]
        dh = flip_terms(pre, unit_terms(G, W["W2"], cells, units))
        slices.append((cells, units, dh, zq))
    units = np.concatenate([sl[1] for sl in slices])
    dh = np.concatenate([sl[2] for sl in slices])
    vec = np.concatenate([sl[2][:, None] * sl[3][sl[0]] for sl in slices]).reshape(-1, c_z)
    chosen = fit_flips(got_dW1 - ref["W1"], units, vec)
    np.add.at(ref["W1"], units[chosen], vec[chosen])
    g_s = np.zeros_like(x)
    at = 0
    for k, (cells, u, h, _) in enumerate(slices):
        pick = chosen[at:at + len(cells)]
        at += len(cells)
        dgz = np.zeros((int(np.square(np.asarray(lengths, dtype=np.int64)).sum()), c_z))
        np.add.at(dgz, cells[pick], h[pick, None] * W["W1"][u[pick]])
        ga, gb = oracle.broadcast_backward(lengths, lengths, dgz)
        g_s[:, k, :] = ga @ W["Wa"] + gb @ W["Wb"]
        ref["Wa"] = ref["Wa"] + ga.T @ x[:, k, :]
        ref["Wb"] = ref["Wb"] + gb.T @ x[:, k, :]
    ref["s"] = ref["s"] + g_s.reshape(T, -1)
    return ref, int(chosen.sum()), len(units)
