"""Pins of the oracle's gradients and of Equation 5 (DanLing NestedTensor,
Appendix A.1) to facts outside the code under test: a hand-evaluated loss,
the printed sample weights, central finite differences of the whole loss,
adjoint (dot-product) identities, the closed form of an all-active
transition, and PyTorch's autograd on a dense per-sample formulation."""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _weights(rng, c_s, c_z, hidden):
    sh = {"Wa": (c_z, c_s), "Wb": (c_z, c_s), "W1": (hidden, c_z), "W2": (c_z, hidden),
          "Wo": (c_s, c_z)}
    return {k: rng.normal(0.0, 1.0 / np.sqrt(v[1]), v) for k, v in sh.items()}


def test_loss_weights_printed_formula():
    # alpha_i = 1 + i/B, beta_i = 1.5 - i/(2B), evaluated by hand for B = 4
    a, b = oracle.loss_weights(4)
    np.testing.assert_array_equal(a, [1.0, 1.25, 1.5, 1.75])
    np.testing.assert_array_equal(b, [1.5, 1.375, 1.25, 1.125])


def test_eq5_hand_computed():
    # B = 2, N = (1, 2), C = C_p = 1: singles 1 | 2, 3 and pair cells 1 | 1, 1, 1, 1.
    # alpha = (1, 1.5), beta = (1.5, 1.25); sum N = 3, sum N^2 = 5.
    # L = (1*1 + 1.5*(4 + 9)) / 3 + (1.5*1 + 1.25*4) / 5 = 20.5/3 + 1.3
    x = np.array([[1.0], [2.0], [3.0]])
    pz = np.ones((5, 1))
    L, gx, gp = oracle.loss_eq5([1, 2], [1, 2], x, pz)
    assert L == pytest.approx(20.5 / 3 + 1.3, rel=1e-15)
    np.testing.assert_allclose(gx[:, 0], [2 / 3, 2.0, 3.0], rtol=1e-15)
    np.testing.assert_allclose(gp[:, 0], [0.6, 0.5, 0.5, 0.5, 0.5], rtol=1e-15)
    # S = 3 (the non-leading layout: each row holds S slices of C values):
    # the same values in every slice give the same loss, and each of the
    # three copies of a value gets a third of its gradient
    L3, gx3, gp3 = oracle.loss_eq5([1, 2], [1, 2], np.repeat(x, 3, axis=1),
                                   np.repeat(pz, 3, axis=1), S=3)
    assert L3 == pytest.approx(L, rel=1e-15)
    np.testing.assert_allclose(gx3, np.repeat(gx / 3, 3, axis=1), rtol=1e-15)
    np.testing.assert_allclose(gp3, np.repeat(gp / 3, 3, axis=1), rtol=1e-15)


def test_eq5_rectangular_divides_by_n_times_m():
    # one sample (B = 1: alpha_0 = 1, beta_0 = 1.5), N = 1, M = 4, C = 2, C_p = 1
    x = np.array([[1.0, 1.0]])
    pz = np.array([[2.0], [0.0], [0.0], [0.0]])
    L, _, _ = oracle.loss_eq5([1], [4], x, pz)
    assert L == pytest.approx(2.0 / 2 + 1.5 * 4.0 / 4, rel=1e-15)


def _fd_check(f, params, grads, h=1e-6, rtol=2e-6):
    """Central differences of the scalar f over every entry of params."""
    for name, arr in params.items():
        g = grads[name]
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            fp = f()
            arr[idx] = keep - h
            fm = f()
            arr[idx] = keep
            num = (fp - fm) / (2 * h)
            scale = max(1.0, float(np.max(np.abs(g))))
            assert abs(num - g[idx]) <= rtol * scale, (name, idx, num, g[idx])


@pytest.mark.parametrize("lengths,seed", [([2, 3, 1], 0), ([4, 1], 1), ([3, 0, 2], 2)])
def test_chain_gradients_match_finite_differences(lengths, seed):
    rng = np.random.default_rng(seed)
    c_s, c_z, hidden = 4, 3, 5
    s = rng.normal(size=(sum(lengths), c_s))
    ws = [_weights(rng, c_s, c_z, hidden) for _ in range(2)]
    L, g_s, grads = oracle.chain_backward(lengths, s, ws)
    assert L == pytest.approx(oracle.chain_loss(lengths, s, ws), rel=1e-14)
    params = {"s": s}
    flat = {"s": g_s}
    for k, (w, g) in enumerate(zip(ws, grads)):
        for name in w:
            params[f"{name}{k}"] = w[name]
            flat[f"{name}{k}"] = g[name]
    _fd_check(lambda: oracle.chain_loss(lengths, s, ws), params, flat)


def test_adjoints_of_broadcast_and_mean():
    # <broadcast(a, b), G> = <a, g_a> + <b, g_b> and <mean(z), g> = <z, mean^T(g)>
    rng = np.random.default_rng(3)
    rows, cols, C = [3, 0, 5, 2], [4, 2, 1, 6], 7
    a = rng.normal(size=(sum(rows), C))
    b = rng.normal(size=(sum(cols), C))
    cells = int(np.dot(rows, cols))
    G = rng.normal(size=(cells, C))
    g_a, g_b = oracle.broadcast_backward(rows, cols, G)
    lhs = float(np.sum(oracle.broadcast_rect(rows, cols, a, b) * G))
    assert lhs == pytest.approx(float(np.sum(a * g_a) + np.sum(b * g_b)), rel=1e-12)
    z = rng.normal(size=(cells, C))
    gm = rng.normal(size=(sum(rows), C))
    lhs = float(np.sum(oracle.reduce_mean_rect(rows, cols, z) * gm))
    rhs = float(np.sum(z * oracle.reduce_mean_backward(rows, cols, gm)))
    assert lhs == pytest.approx(rhs, rel=1e-12)


def test_transition_all_active_is_linear():
    # with every pre-activation positive the map is z -> z + z W1^T W2^T, whose
    # adjoint is G (I + W2 W1) and whose weight gradients are G^T (z W1^T) and
    # (G W2)^T z
    rng = np.random.default_rng(4)
    z = rng.uniform(0.1, 1.0, (9, 4))
    W1 = rng.uniform(0.1, 1.0, (6, 4))
    W2 = rng.normal(size=(4, 6))
    G = rng.normal(size=(9, 4))
    g_z, dW1, dW2 = oracle.transition_backward(z, W1, W2, G)
    np.testing.assert_allclose(g_z, G @ (np.eye(4) + W2 @ W1), rtol=1e-12)
    np.testing.assert_allclose(dW2, G.T @ (z @ W1.T), rtol=1e-12)
    np.testing.assert_allclose(dW1, (G @ W2).T @ z, rtol=1e-12)


def test_chain_gradients_match_torch_autograd_dense():
    """A dense per-sample formulation (each sample its own N x N pair block,
    no packing) differentiated by PyTorch's autograd in float64."""
    rng = np.random.default_rng(5)
    lengths, c_s, c_z, hidden = [5, 9, 3], 8, 6, 10
    s = rng.normal(size=(sum(lengths), c_s))
    ws = [_weights(rng, c_s, c_z, hidden) for _ in range(2)]
    L, g_s, grads = oracle.chain_backward(lengths, s, ws)

    ts = torch.tensor(s, requires_grad=True)
    tw = [{k: torch.tensor(v, requires_grad=True) for k, v in w.items()} for w in ws]
    B = len(lengths)
    xs = list(torch.split(ts, lengths))
    for w in tw:
        new_x, pairs = [], []
        for X in xs:
            P = (X @ w["Wa"].T)[:, None, :] + (X @ w["Wb"].T)[None, :, :]
            P = P + torch.relu(P @ w["W1"].T) @ w["W2"].T
            new_x.append(X + P.mean(dim=1) @ w["Wo"].T)
            pairs.append(P)
        xs = new_x
    n = torch.tensor(lengths, dtype=torch.float64)
    alpha = 1 + torch.arange(B, dtype=torch.float64) / B
    beta = 1.5 - torch.arange(B, dtype=torch.float64) / (2 * B)
    t1 = sum(alpha[i] * (xs[i] ** 2).sum() for i in range(B)) / (c_s * n.sum())
    t2 = sum(beta[i] * (pairs[i] ** 2).sum() for i in range(B)) / (c_z * (n * n).sum())
    loss = t1 + t2
    loss.backward()
    assert float(loss.detach()) == pytest.approx(L, rel=1e-12)
    np.testing.assert_allclose(ts.grad.numpy(), g_s, rtol=1e-10, atol=1e-13)
    for w, g in zip(tw, grads):
        for k in w:
            np.testing.assert_allclose(w[k].grad.numpy(), g[k], rtol=1e-10, atol=1e-13)


def test_non_leading_block_is_per_slice_leading_block():
    """Nothing in the block mixes the static axis: slice k of the non-leading
    block equals the leading block on slice k of the singles."""
    rng = np.random.default_rng(8)
    lengths, S, c_s, c_z, hidden = [3, 0, 5, 2], 3, 4, 6, 5
    s = rng.normal(size=(sum(lengths), S * c_s))
    w = _weights(rng, c_s, c_z, hidden)
    s_out, z_out = oracle.block_nl(lengths, s, w, S)
    cells = int(np.square(lengths).sum())
    for k in range(S):
        rs, rz = oracle.block(lengths, s[:, k * c_s:(k + 1) * c_s], w)
        np.testing.assert_allclose(s_out[:, k * c_s:(k + 1) * c_s], rs, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(z_out.reshape(cells, S, c_z)[:, k, :], rz, rtol=1e-12,
                                   atol=1e-12)


def test_non_leading_gradients_match_finite_differences():
    rng = np.random.default_rng(9)
    lengths, S, c_s, c_z, hidden = [2, 3], 3, 4, 3, 5
    s = rng.normal(size=(sum(lengths), S * c_s))
    w = _weights(rng, c_s, c_z, hidden)

    def loss():
        so, zo = oracle.block_nl(lengths, s, w, S)
        return oracle.loss_eq5(lengths, lengths, so, zo, S=S)[0]

    so, zo = oracle.block_nl(lengths, s, w, S)
    _, gx, gz = oracle.loss_eq5(lengths, lengths, so, zo, S=S)
    g = oracle.block_backward_nl(lengths, s, w, S, gx, gz)
    params = {"s": s, **w}
    _fd_check(loss, params, g)


# ------------------------------------------------ the SwiGLU block (Eq. 1)
def _swiglu_weights(rng, c_s, c_z, hidden):
    return {"Wa": rng.normal(0.0, 1.0 / np.sqrt(c_s), (c_z, c_s)),
            "Wb": rng.normal(0.0, 1.0 / np.sqrt(c_s), (c_z, c_s)),
            "Wo": rng.normal(0.0, 1.0 / np.sqrt(c_z), (c_s, c_z)),
            "ln_gamma": 1.0 + 0.3 * rng.normal(size=c_z),
            "ln_beta": 0.2 * rng.normal(size=c_z),
            "Wg": rng.normal(0.0, 1.0 / np.sqrt(c_z), (hidden, c_z)),
            "Wu": rng.normal(0.0, 1.0 / np.sqrt(c_z), (hidden, c_z)),
            "Wd": rng.normal(0.0, 1.0 / np.sqrt(hidden), (c_z, hidden))}


@pytest.mark.parametrize("lengths,seed", [([2, 3, 1], 10), ([3, 0, 2], 11)])
def test_swiglu_chain_gradients_match_finite_differences(lengths, seed):
    rng = np.random.default_rng(seed)
    c_s, c_z, hidden = 4, 3, 5
    s = rng.normal(size=(sum(lengths), c_s))
    ws = [_swiglu_weights(rng, c_s, c_z, hidden) for _ in range(2)]
    L, g_s, grads = oracle.chain_swiglu_backward(lengths, s, ws)
    assert L == pytest.approx(oracle.chain_swiglu_loss(lengths, s, ws), rel=1e-14)
    params = {"s": s}
    flat = {"s": g_s}
    for k, (w, g) in enumerate(zip(ws, grads)):
        for name in w:
            params[f"{name}{k}"] = w[name]
            flat[f"{name}{k}"] = g[name]
    _fd_check(lambda: oracle.chain_swiglu_loss(lengths, s, ws), params, flat)


def test_layer_norm_adjoint_identities():
    # LN(z + c 1) = LN(z) and LN(k z) = LN(z) (eps = 0): the adjoint of every
    # row is orthogonal to the ones vector and to the row itself; with the
    # plain mean removed, <g_z, dz> equals <g_x, d LN> for any direction dz
    rng = np.random.default_rng(12)
    z = rng.normal(size=(7, 9))
    gamma, gx = 1 + rng.normal(size=9), rng.normal(size=(7, 9))
    g_z, dgamma, dbeta = oracle.layer_norm_backward(z, gamma, gx, 0.0)
    np.testing.assert_allclose(g_z.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((g_z * z).sum(axis=1), 0.0, atol=1e-11)
    dz = rng.normal(size=z.shape)
    h = 1e-6
    dx = (oracle.layer_norm(z + h * dz, gamma, 0 * gamma, 0.0)
          - oracle.layer_norm(z - h * dz, gamma, 0 * gamma, 0.0)) / (2 * h)
    assert float((g_z * dz).sum()) == pytest.approx(float((gx * dx).sum()), rel=1e-7)
    xhat = oracle.layer_norm(z, np.ones(9), np.zeros(9), 0.0)
    np.testing.assert_allclose(dgamma, (gx * xhat).sum(axis=0), rtol=1e-12)
    np.testing.assert_allclose(dbeta, gx.sum(axis=0), rtol=1e-12)


def test_swiglu_transition_zero_down_weights():
    # Wd = 0: the transition is the identity, so g_z = G and every weight of
    # the gate and the LN gets no gradient; dWd is G^T (silu(g) * u)
    rng = np.random.default_rng(13)
    z, G = rng.normal(size=(11, 6)), rng.normal(size=(11, 6))
    gamma, beta = 1 + rng.normal(size=6), rng.normal(size=6)
    Wg, Wu = rng.normal(size=(8, 6)), rng.normal(size=(8, 6))
    g_z, dga, dbe, dWg, dWu, dWd = oracle.transition_swiglu_backward(
        z, gamma, beta, Wg, Wu, np.zeros((6, 8)), G)
    np.testing.assert_array_equal(g_z, G)
    for v in (dga, dbe, dWg, dWu):
        np.testing.assert_array_equal(v, 0.0)
    x = oracle.layer_norm(z, gamma, beta, 1e-5)
    g = x @ Wg.T
    np.testing.assert_allclose(dWd, G.T @ (g / (1 + np.exp(-g)) * (x @ Wu.T)), rtol=1e-12)


def test_swiglu_chain_gradients_match_torch_autograd_dense():
    """Dense per-sample SwiGLU blocks (LN and silu from torch.nn.functional)
    differentiated by PyTorch's autograd in float64."""
    F = torch.nn.functional
    rng = np.random.default_rng(14)
    lengths, c_s, c_z, hidden = [5, 9, 3], 8, 6, 12
    s = rng.normal(size=(sum(lengths), c_s))
    ws = [_swiglu_weights(rng, c_s, c_z, hidden) for _ in range(2)]
    L, g_s, grads = oracle.chain_swiglu_backward(lengths, s, ws)
    ts = torch.tensor(s, requires_grad=True)
    tw = [{k: torch.tensor(v, requires_grad=True) for k, v in w.items()} for w in ws]
    B = len(lengths)
    xs = list(torch.split(ts, lengths))
    for w in tw:
        new_x, pairs = [], []
        for X in xs:
            P = (X @ w["Wa"].T)[:, None, :] + (X @ w["Wb"].T)[None, :, :]
            x = F.layer_norm(P, (c_z,), w["ln_gamma"], w["ln_beta"], eps=1e-5)
            P = P + (F.silu(x @ w["Wg"].T) * (x @ w["Wu"].T)) @ w["Wd"].T
            new_x.append(X + P.mean(dim=1) @ w["Wo"].T)
            pairs.append(P)
        xs = new_x
    n = torch.tensor(lengths, dtype=torch.float64)
    alpha = 1 + torch.arange(B, dtype=torch.float64) / B
    beta = 1.5 - torch.arange(B, dtype=torch.float64) / (2 * B)
    loss = sum(alpha[i] * (xs[i] ** 2).sum() for i in range(B)) / (c_s * n.sum()) \
        + sum(beta[i] * (pairs[i] ** 2).sum() for i in range(B)) / (c_z * (n * n).sum())
    loss.backward()
    assert float(loss.detach()) == pytest.approx(L, rel=1e-12)
    np.testing.assert_allclose(ts.grad.numpy(), g_s, rtol=1e-10, atol=1e-13)
    for w, g in zip(tw, grads):
        for k in w:
            np.testing.assert_allclose(w[k].grad.numpy(), g[k], rtol=1e-10, atol=1e-13)
