"""Plain float64 gradients of the packed single-pair-single block and the
sample-weighted squared loss it is trained with.

TEST INFRASTRUCTURE (see the package docstring): callers are tests/, the
smoke check and the CPU-baseline leg of the benchmark only.

Source: the DanLing NestedTensor paper (arXiv 2609.30379).

* Appendix A.1, Equation 5 - the objective over the returned singles X~ and
  pair state P~: L = sum_i alpha_i |X~_i|_F^2 / (S C sum_i N_i)
  + sum_i beta_i |P~_i|_F^2 / (S C_p sum_i N_i M_i), with
  alpha_i = 1 + i / B and beta_i = 1.5 - i / (2 B) for i = 0 .. B - 1, S = 1
  for the leading layouts, M_i = N_i for square pairs. The squared sums
  accumulate in at least fp32 (here fp64).
* Section 4 (experimental setup) - the measured step is forward, loss and
  backward; Section 3.4 - gradients must reach the projections, the pair
  update and the reduction of Equation 1 through the packed storage.

The backward pass is the chain rule applied to the forward of pair_block,
step by step in reverse order, written from the forward's definitions:

  forward                          adjoint (g_x = dL/dx)
  a = s Wa^T, b = s Wb^T           g_s += g_a Wa + g_b Wb; dWa = g_a^T s; dWb = g_b^T s
  z[o_i + r N_i + c] = a[r] + b[c] g_a[r] = sum_c g_z[..];   g_b[c] = sum_r g_z[..]
  P = relu(z W1^T)                 G = g_z' ; g_P = G W2 ; dW2 = G^T P
  z' = z + P W2^T                  g_H = g_P * [z W1^T > 0]; dW1 = g_H^T z
                                   g_z = G + g_H W1
  m[r] = (1/M_i) sum_c z'[..]      G[o_i + r M_i + c] += g_m[r] / M_i
  s~ = s + m Wo^T                  g_m = g_s~ Wo; dWo = g_s~^T m; g_s = g_s~ + ...

The block with the paper's own transition (pre-normalised SwiGLU,
pair_block.block_swiglu) has its gradients here too: the chain rule through
the SwiGLU gate, its three products and the LayerNorm over the c_z features.

Pins (tests/test_oracle_backward_pins.py): central finite differences of the
whole loss through two-block chains (ReLU and SwiGLU), a hand-evaluated
Equation 5, adjoint (dot-product) identities of the broadcast and the mean,
LayerNorm's adjoint identities, the closed forms of an all-active ReLU
transition and of a SwiGLU transition with zero output weights, and
PyTorch's autograd on dense per-sample formulations.
"""
from __future__ import annotations

import numpy as np

from .pair_block import (_CHUNK_ROWS, block, block_swiglu, broadcast, layer_norm, project,
                         reduce_mean, transition)


# ------------------------------------------------------------------ Eq. 5
def loss_weights(B):
    """alpha_i = 1 + i / B and beta_i = 1.5 - i / (2 B), i = 0 .. B - 1."""
    i = np.arange(B, dtype=np.float64)
    return 1.0 + i / B, 1.5 - i / (2.0 * B)


def loss_eq5(rows, cols, x, pz, S=1):
    """Equation 5 over the singles x [sum N_i, S*C] and the pair state
    pz [sum N_i M_i, S*C_p]; S is the static leading axis of the non-leading
    layout, packed inside each row (Eq. 2 moves the ragged axes to the
    front), so ||X_i||_F^2 sums S*N_i*C values and S = 1 is the leading
    layout. Returns (L, g_x, g_pz) with the exact gradients
    g_x = 2 alpha_i x / (S C sum N) and g_pz = 2 beta_i pz / (S C_p sum N M)."""
    x = np.asarray(x, dtype=np.float64)
    pz = np.asarray(pz, dtype=np.float64)
    N = [int(n) for n in rows]
    M = [int(m) for m in cols]
    B = len(N)
    alpha, beta = loss_weights(B)
    if x.shape[1] % S or pz.shape[1] % S:
        raise ValueError("row widths must be multiples of S")
    C, Cp = x.shape[1] // S, pz.shape[1] // S
    d1 = S * C * sum(N)
    d2 = S * Cp * sum(n * m for n, m in zip(N, M))
    L = 0.0
    g_x = np.zeros_like(x)
    g_pz = np.zeros_like(pz)
    r0 = c0 = 0
    for i in range(B):
        xi = x[r0:r0 + N[i]]
        pi = pz[c0:c0 + N[i] * M[i]]
        if d1:
            L += alpha[i] * float(np.sum(xi * xi)) / d1
            g_x[r0:r0 + N[i]] = 2.0 * alpha[i] * xi / d1
        if d2:
            L += beta[i] * float(np.sum(pi * pi)) / d2
            g_pz[c0:c0 + N[i] * M[i]] = 2.0 * beta[i] * pi / d2
        r0 += N[i]
        c0 += N[i] * M[i]
    return L, g_x, g_pz


# ------------------------------------------------------------- adjoints
def reduce_mean_backward(rows, cols, g_m):
    """Adjoint of the column mean (Eq. 4 divided by M_i): every cell of pair
    row r of sample i receives g_m[eta_i + r] / M_i."""
    g_m = np.asarray(g_m, dtype=np.float64)
    out = []
    r0 = 0
    for n, m in zip((int(v) for v in rows), (int(v) for v in cols)):
        blk = g_m[r0:r0 + n]
        if m:
            out.append(np.repeat(blk / m, m, axis=0))
        r0 += n
    if not out:
        return np.zeros((0, g_m.shape[1]))
    return np.concatenate(out, axis=0)


def broadcast_backward(rows, cols, g_z):
    """Adjoint of z[o_i + r M_i + c] = a[eta_i + r] + b[mu_i + c]: g_a sums a
    sample's pair rows over their columns, g_b its pair columns over rows."""
    g_z = np.asarray(g_z, dtype=np.float64)
    C = g_z.shape[1]
    N = [int(n) for n in rows]
    M = [int(m) for m in cols]
    g_a = np.zeros((sum(N), C))
    g_b = np.zeros((sum(M), C))
    r0 = c0 = o = 0
    for n, m in zip(N, M):
        blk = g_z[o:o + n * m].reshape(n, m, C)
        g_a[r0:r0 + n] = blk.sum(axis=1)
        g_b[c0:c0 + m] = blk.sum(axis=0)
        r0 += n
        c0 += m
        o += n * m
    return g_a, g_b


def transition_backward(z, W1, W2, G):
    """Gradients of z' = z + relu(z W1^T) W2^T for an incoming G = dL/dz'.
    Returns (g_z, dW1, dW2). The derivative of relu at 0 is taken as 0."""
    z = np.asarray(z, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    g_z = np.empty_like(z)
    dW1 = np.zeros_like(W1)
    dW2 = np.zeros_like(W2)
    for s in range(0, z.shape[0], _CHUNK_ROWS):
        zc, Gc = z[s:s + _CHUNK_ROWS], G[s:s + _CHUNK_ROWS]
        pre = zc @ W1.T
        P = np.maximum(pre, 0.0)
        g_H = (Gc @ W2) * (pre > 0.0)
        dW2 += Gc.T @ P
        dW1 += g_H.T @ zc
        g_z[s:s + _CHUNK_ROWS] = Gc + g_H @ W1
    return g_z, dW1, dW2


def layer_norm_backward(z, gamma, g_x, eps):
    """Adjoint of x = xhat * gamma + beta, xhat = (z - mean) / sqrt(var + eps)
    over the features of each row (biased variance), for an incoming g_x.
    With g_xhat = g_x * gamma, the mean's and the variance's dependence on
    every feature give g_z = (g_xhat - mean(g_xhat) - xhat mean(g_xhat xhat))
    / sqrt(var + eps); dgamma = sum over rows of g_x xhat, dbeta = sum of
    g_x. Returns (g_z, dgamma, dbeta)."""
    z = np.asarray(z, dtype=np.float64)
    g_x = np.asarray(g_x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    mu = z.mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(np.square(z - mu).mean(axis=-1, keepdims=True) + eps)
    xhat = (z - mu) * rstd
    gh = g_x * gamma
    g_z = rstd * (gh - gh.mean(axis=-1, keepdims=True)
                  - xhat * (gh * xhat).mean(axis=-1, keepdims=True))
    return g_z, (g_x * xhat).sum(axis=0), g_x.sum(axis=0)


def transition_swiglu_backward(z, gamma, beta, Wg, Wu, Wd, G, eps=1e-5):
    """Gradients of z' = z + (silu(x Wg^T) * (x Wu^T)) Wd^T, x = LN(z), for an
    incoming G = dL/dz'. With g = x Wg^T, u = x Wu^T, s = sigmoid(g) and the
    gated activation A = g s u:
      dWd = G^T A,  g_A = G Wd,
      g_u = g_A g s,  g_g = g_A u s (1 + g (1 - s))   (silu' = s (1 + g (1 - s))),
      dWu = g_u^T x,  dWg = g_g^T x,  g_x = g_u Wu + g_g Wg,
      g_z = G + LN's adjoint of g_x (layer_norm_backward).
    Returns (g_z, dgamma, dbeta, dWg, dWu, dWd)."""
    z = np.asarray(z, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    Wg, Wu, Wd = (np.asarray(w, dtype=np.float64) for w in (Wg, Wu, Wd))
    g_z = np.empty_like(z)
    dWg, dWu, dWd = np.zeros_like(Wg), np.zeros_like(Wu), np.zeros_like(Wd)
    dgamma = np.zeros(z.shape[1])
    dbeta = np.zeros(z.shape[1])
    for c in range(0, z.shape[0], _CHUNK_ROWS):
        zc, Gc = z[c:c + _CHUNK_ROWS], G[c:c + _CHUNK_ROWS]
        x = layer_norm(zc, gamma, beta, eps)
        g = x @ Wg.T
        u = x @ Wu.T
        sg = 1.0 / (1.0 + np.exp(-g))
        A = g * sg * u
        dWd += Gc.T @ A
        gA = Gc @ Wd
        gu = gA * g * sg
        gg = gA * u * sg * (1.0 + g * (1.0 - sg))
        dWu += gu.T @ x
        dWg += gg.T @ x
        gzl, dga, dbe = layer_norm_backward(zc, gamma, gu @ Wu + gg @ Wg, eps)
        g_z[c:c + _CHUNK_ROWS] = Gc + gzl
        dgamma += dga
        dbeta += dbe
    return g_z, dgamma, dbeta, dWg, dWu, dWd


# ------------------------------------------------------------- the block
def block_backward(lengths, s, w, g_s_out, g_z_out=None):
    """Gradients of one square block (pair_block.block) for incoming g_s_out
    = dL/ds~ and, optionally, g_z_out = dL/dz' (the returned pair state).
    Returns a dict with "s" (dL/ds) and "Wa", "Wb", "W1", "W2", "Wo"."""
    s = np.asarray(s, dtype=np.float64)
    g_s_out = np.asarray(g_s_out, dtype=np.float64)
    W = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    # forward, keeping what the adjoints read
    a = project(s, W["Wa"])
    b = project(s, W["Wb"])
    z = broadcast(lengths, a, b)
    zt = transition(z, W["W1"], W["W2"])
    m = reduce_mean(lengths, zt)
    # s~ = s + m Wo^T
    g_m = g_s_out @ W["Wo"]
    dWo = g_s_out.T @ m
    G = reduce_mean_backward(lengths, lengths, g_m)
    if g_z_out is not None:
        G = G + np.asarray(g_z_out, dtype=np.float64)
    g_z, dW1, dW2 = transition_backward(z, W["W1"], W["W2"], G)
    g_a, g_b = broadcast_backward(lengths, lengths, g_z)
    g_s = g_s_out + g_a @ W["Wa"] + g_b @ W["Wb"]
    return {"s": g_s, "Wa": g_a.T @ s, "Wb": g_b.T @ s, "W1": dW1, "W2": dW2, "Wo": dWo}


def block_swiglu_backward(lengths, s, w, g_s_out, g_z_out=None, eps=1e-5):
    """Gradients of pair_block.block_swiglu for incoming g_s_out and,
    optionally, g_z_out: the steps of block_backward with the SwiGLU
    transition's adjoint. Returns a dict with "s" and the gradient of every
    weight (Wa, Wb, Wo, ln_gamma, ln_beta, Wg, Wu, Wd)."""
    s = np.asarray(s, dtype=np.float64)
    g_s_out = np.asarray(g_s_out, dtype=np.float64)
    W = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    a = project(s, W["Wa"])
    b = project(s, W["Wb"])
    z = broadcast(lengths, a, b)
    zt = block_swiglu(lengths, s, W, eps)[1]
    m = reduce_mean(lengths, zt)
    g_m = g_s_out @ W["Wo"]
    dWo = g_s_out.T @ m
    G = reduce_mean_backward(lengths, lengths, g_m)
    if g_z_out is not None:
        G = G + np.asarray(g_z_out, dtype=np.float64)
    g_z, dga, dbe, dWg, dWu, dWd = transition_swiglu_backward(
        z, W["ln_gamma"], W["ln_beta"], W["Wg"], W["Wu"], W["Wd"], G, eps)
    g_a, g_b = broadcast_backward(lengths, lengths, g_z)
    g_s = g_s_out + g_a @ W["Wa"] + g_b @ W["Wb"]
    return {"s": g_s, "Wa": g_a.T @ s, "Wb": g_b.T @ s, "Wo": dWo, "ln_gamma": dga,
            "ln_beta": dbe, "Wg": dWg, "Wu": dWu, "Wd": dWd}


def chain_swiglu_loss(lengths, s, ws, eps=1e-5):
    """Equation 5 of a chain of SwiGLU blocks."""
    z = None
    x = np.asarray(s, dtype=np.float64)
    for w in ws:
        x, z = block_swiglu(lengths, x, w, eps)
    return loss_eq5(lengths, lengths, x, z)[0]


def chain_swiglu_backward(lengths, s, ws, eps=1e-5):
    """Loss and gradients of a chain of SwiGLU blocks under Equation 5.
    Returns (L, g_s, [per-block weight gradients])."""
    xs = [np.asarray(s, dtype=np.float64)]
    z = None
    for w in ws:
        x, z = block_swiglu(lengths, xs[-1], w, eps)
        xs.append(x)
    L, g_x, g_z = loss_eq5(lengths, lengths, xs[-1], z)
    grads = [None] * len(ws)
    g = g_x
    for k in range(len(ws) - 1, -1, -1):
        r = block_swiglu_backward(lengths, xs[k], ws[k], g, g_z if k == len(ws) - 1 else None,
                                  eps)
        g = r.pop("s")
        grads[k] = r
    return L, g, grads


def chain_loss(lengths, s, ws, S=1):
    """Equation 5 of a chain of blocks: the loss reads the last block's singles
    and pair state. Returns the scalar loss."""
    z = None
    x = np.asarray(s, dtype=np.float64)
    for w in ws:
        x, z = block(lengths, x, w)
    L, _, _ = loss_eq5(lengths, lengths, x, z, S)
    return L


def chain_backward(lengths, s, ws, S=1):
    """Loss and gradients of a chain of square blocks under Equation 5.
    Returns (L, g_s, [per-block weight gradients])."""
    xs = [np.asarray(s, dtype=np.float64)]
    z = None
    for w in ws:
        x, z = block(lengths, xs[-1], w)
        xs.append(x)
    L, g_x, g_z = loss_eq5(lengths, lengths, xs[-1], z, S)
    grads = [None] * len(ws)
    g = g_x
    for k in range(len(ws) - 1, -1, -1):
        r = block_backward(lengths, xs[k], ws[k], g, g_z if k == len(ws) - 1 else None)
        g = r.pop("s")
        grads[k] = r
    return L, g, grads


# --------------------------------------------- non-leading layout (S, N_i, C)
def block_nl(lengths, s, w, S):
    """The block on the non-leading layout: each sample's singles are
    (S, N_i, C), packed as rows of S*C values (Eq. 2), its pair state
    (S, N_i, N_i, C_p) as rows of S*C_p. Projections, the transition and the
    output projection act on the last axis, the broadcast adds along the pair
    axes, the mean runs over columns: nothing mixes the S slices. Written
    with an explicit S axis. Returns (s_out [T, S*c_s], z_out [cells, S*c_z])."""
    s = np.asarray(s, dtype=np.float64)
    T = s.shape[0]
    x = s.reshape(T, S, -1)
    W = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    a = x @ W["Wa"].T                      # [T, S, c_z]
    b = x @ W["Wb"].T
    c_z = a.shape[2]
    zs, ms = [], []
    eta = 0
    for n in (int(v) for v in lengths):
        A, Bm = a[eta:eta + n], b[eta:eta + n]              # [n, S, c_z]
        Z = A[:, None, :, :] + Bm[None, :, :, :]            # [n, n, S, c_z]
        Z = Z + np.maximum(Z @ W["W1"].T, 0.0) @ W["W2"].T
        zs.append(Z.reshape(n * n, S * c_z))
        if n:
            ms.append(Z.mean(axis=1))                       # [n, S, c_z]
        eta += n
    z = np.concatenate(zs, axis=0) if zs else np.zeros((0, S * c_z))
    m = np.concatenate(ms, axis=0) if ms else np.zeros((0, S, c_z))
    out = x + m @ W["Wo"].T
    return out.reshape(T, -1), z


def block_backward_nl(lengths, s, w, S, g_s_out, g_z_out=None):
    """Gradients of block_nl: the S slices are independent blocks sharing the
    weights, so the single and pair gradients are per slice and the weight
    gradients are sums over slices (the chain rule through the shared
    weights). Returns a dict like block_backward."""
    s = np.asarray(s, dtype=np.float64)
    T = s.shape[0]
    x = s.reshape(T, S, -1)
    gs = np.asarray(g_s_out, dtype=np.float64).reshape(T, S, -1)
    gz = None if g_z_out is None else np.asarray(g_z_out, dtype=np.float64)
    c_z = np.asarray(w["Wa"]).shape[0]
    out = {"s": np.zeros_like(x)}
    for k in range(S):
        gzk = None if gz is None else gz.reshape(gz.shape[0], S, c_z)[:, k, :]
        r = block_backward(lengths, x[:, k, :], w, gs[:, k, :], gzk)
        out["s"][:, k, :] = r.pop("s")
        for name, v in r.items():
            out[name] = out.get(name, 0.0) + v
    out["s"] = out["s"].reshape(T, -1)
    return out
