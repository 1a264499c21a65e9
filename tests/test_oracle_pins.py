"""Pins of the CPU oracle against facts outside itself (no GPU needed).

Each test ties an oracle function to a printed value of the DanLing
NestedTensor paper, a hand-computed example, a closed form, an independent
formulation (scalar loops, padded-then-masked, gather indices) or an
invariance the method must have (sample locality, Appendix A).
"""
import json
import os

import numpy as np
import pytest

import oracle
import pair_inputs as pin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _w64(w):
    return {k: v.f64 for k, v in w.items()}


# --------------------------------------------------------------- structure
def test_fig2_partition_printed_and_derived():
    g = _load("fig2_partition.json")
    pr, dv = g["printed"], g["derived_by_hand_from_eq3"]
    p = oracle.partition(pr["lengths"])
    assert p["T"] == pr["T"] and p["cells"] == pr["cells"]
    assert p["single_offsets"].tolist() == pr["single_offsets"]
    assert p["pair_offsets"].tolist() == pr["pair_offsets"]
    assert len(p["row_splits"]) == pr["row_split_entries"]
    assert p["row_splits"].tolist() == dv["row_splits"]
    assert p["row_sample"].tolist() == dv["row_sample"]
    # first-level pair splits (rows per sample) differ from pair sample offsets
    assert p["single_offsets"].tolist() != p["pair_offsets"].tolist()
    smp, row, col = oracle.decode_cells(pr["lengths"])
    assert smp.tolist() == dv["cell_sample"]
    assert row.tolist() == dv["cell_row"]
    assert col.tolist() == dv["cell_col"]


@pytest.mark.parametrize("lengths", [[3, 0, 0, 5, 1], [0], [], [4], [0, 0, 2, 0]])
def test_appendix_a_invariants(lengths):
    p = oracle.partition(lengths)
    o, eta = p["pair_offsets"], p["single_offsets"]
    assert o[0] == 0 and eta[0] == 0
    assert np.diff(o).tolist() == [n * n for n in lengths]
    assert np.diff(eta).tolist() == list(lengths)
    assert o[-1] == p["cells"] == sum(n * n for n in lengths)
    assert eta[-1] == p["T"] == sum(lengths)
    assert len(p["row_splits"]) == 1 + sum(lengths)
    # zero-volume samples have coincident consecutive offsets
    for i, n in enumerate(lengths):
        if n == 0:
            assert o[i] == o[i + 1] and eta[i] == eta[i + 1]


def test_workload_totals():
    # cell totals stated with the workloads: 474 for the tiny case, ~1.79M for the long one
    assert oracle.partition(pin.workload_inputs(0).lengths)["cells"] == 474
    assert oracle.partition(pin.workload_inputs(4).lengths)["cells"] == 1_795_072


def test_decode_is_a_bijection_and_inverts_row_splits():
    rng = np.random.default_rng(7)
    lengths = rng.integers(0, 9, 12).tolist() + [0, 1]
    p = oracle.partition(lengths)
    smp, row, col = oracle.decode_cells(lengths)
    assert (smp >= 0).all()  # every cell hit
    # enumerating (i, r, c) in batch/row-major order visits each cell once, in order
    ell = []
    for i, n in enumerate(lengths):
        for r in range(n):
            for c in range(n):
                ell.append(p["pair_offsets"][i] + r * n + c)
    assert ell == list(range(p["cells"]))
    # independent inversion through the second-level splits
    t = np.arange(p["cells"])
    g = np.searchsorted(p["row_splits"], t, side="right") - 1
    assert (p["row_sample"][g] == smp).all()
    assert (g - p["single_offsets"][smp] == row).all()
    assert (t - p["row_splits"][g] == col).all()


def test_equal_totals_different_partitions():
    # (2,3) and (3,2): both 5 singles and 13 cells, but not the same structure
    p23, p32 = oracle.partition([2, 3]), oracle.partition([3, 2])
    assert p23["T"] == p32["T"] and p23["cells"] == p32["cells"]
    assert p23["pair_offsets"].tolist() != p32["pair_offsets"].tolist()
    x = pin.make_inputs([2, 3], 8, 8, 16, "f32", seed=3)
    w = _w64(x.weights[0])
    s23, _ = oracle.block([2, 3], x.s.f64, w)
    s32, _ = oracle.block([3, 2], x.s.f64, w)
    assert not np.allclose(s23, s32)


# --------------------------------------------------------- worked example
def test_hand_computed_block():
    g = _load("hand_block.json")
    L = g["lengths"]
    s = np.array(g["s"], dtype=np.float64)
    w = {k: np.array(g[k], dtype=np.float64) for k in ("Wa", "Wb", "W1", "W2", "Wo")}
    for fn in (oracle.block, oracle.block_bruteforce, oracle.block_padded_masked,
               oracle.block_gather):
        so, zo = fn(L, s, w)
        assert zo.tolist() == g["z_out"], fn.__name__
        assert so.tolist() == g["s_out"], fn.__name__
    zt = oracle.transition(oracle.broadcast(L, oracle.project(s, w["Wa"]),
                                            oracle.project(s, w["Wb"])), w["W1"], w["W2"])
    assert oracle.reduce_mean(L, zt).tolist() == g["m"]


# ------------------------------------------------------ independent forms
@pytest.mark.parametrize("lengths,seed", [([3, 1, 4], 0), ([2, 0, 5, 1], 1), ([6], 2),
                                          ([1, 1, 1], 3), ([0, 3], 4)])
def test_four_forms_agree(lengths, seed):
    x = pin.make_inputs(lengths, 8, 8, 16, "f32", seed=seed)
    w = _w64(x.weights[0])
    ref_s, ref_z = oracle.block_bruteforce(lengths, x.s.f64, w)
    for fn in (oracle.block, oracle.block_padded_masked, oracle.block_gather):
        so, zo = fn(lengths, x.s.f64, w)
        np.testing.assert_allclose(zo, ref_z, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(so, ref_s, rtol=1e-12, atol=1e-12)


def test_packed_equals_padded_medium():
    lengths = [17, 3, 0, 30, 9]
    x = pin.make_inputs(lengths, 24, 16, 48, "bf16", seed=11)
    w = _w64(x.weights[0])
    s1, z1 = oracle.block(lengths, x.s.f64, w)
    s2, z2 = oracle.block_padded_masked(lengths, x.s.f64, w)
    np.testing.assert_allclose(z1, z2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)


def test_single_sample_equals_dense():
    x = pin.make_inputs([11], 16, 8, 24, "f32", seed=5)
    w = _w64(x.weights[0])
    so, zo = oracle.block([11], x.s.f64, w)
    Xo, Po = oracle.dense_block(x.s.f64, w)
    np.testing.assert_allclose(zo, Po.reshape(-1, 8), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(so, Xo, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------ closed forms
def test_broadcast_single_sample_is_outer_sum():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((5, 3))
    b = rng.standard_normal((5, 3))
    z = oracle.broadcast([5], a, b)
    for r in range(5):
        for c in range(5):
            assert (z[r * 5 + c] == a[r] + b[c]).all()


def test_transition_zero_weights_is_identity():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((40, 8))
    W1 = rng.standard_normal((16, 8))
    W2 = rng.standard_normal((8, 16))
    assert (oracle.transition(z, np.zeros_like(W1), W2) == z).all()
    assert (oracle.transition(z, W1, np.zeros_like(W2)) == z).all()


def test_transition_permutation_weights():
    # W1 = permutation P (hidden h reads feature pi(h)), W2 = identity:
    # z~[f] = z[f] + relu(z[pi(f)]); a transposed W1 would read pi^-1 instead.
    pi = np.array([2, 0, 3, 1])           # not an involution
    P = np.zeros((4, 4))
    P[np.arange(4), pi] = 1.0
    rng = np.random.default_rng(2)
    z = rng.standard_normal((25, 4))
    got = oracle.transition(z, P, np.eye(4))
    assert (got == z + np.maximum(z[:, pi], 0.0)).all()
    inv = np.argsort(pi)
    assert not np.allclose(got, z + np.maximum(z[:, inv], 0.0))


def test_reduce_closed_form_without_transition():
    # W2 = 0: z~ = z, so m[eta_i + r] = a[eta_i + r] + mean_c b[eta_i + c]
    lengths = [4, 0, 7, 1]
    rng = np.random.default_rng(3)
    T = sum(lengths)
    a = rng.standard_normal((T, 5))
    b = rng.standard_normal((T, 5))
    z = oracle.broadcast(lengths, a, b)
    m = oracle.reduce_mean(lengths, z)
    eta = 0
    for n in lengths:
        for r in range(n):
            np.testing.assert_allclose(m[eta + r], a[eta + r] + b[eta:eta + n].mean(axis=0),
                                       rtol=1e-14, atol=1e-14)
        eta += n


def test_reduce_equal_lengths_is_batched_mean():
    rng = np.random.default_rng(4)
    B, n, C = 3, 6, 4
    zt = rng.standard_normal((B * n * n, C))
    m = oracle.reduce_mean([n] * B, zt)
    ref = zt.reshape(B, n, n, C).mean(axis=2).reshape(B * n, C)
    np.testing.assert_allclose(m, ref, rtol=1e-14, atol=1e-14)
    # the row axis would give something else
    assert not np.allclose(m, zt.reshape(B, n, n, C).mean(axis=1).reshape(B * n, C))


def test_reduce_eq4_bruteforce():
    lengths = [3, 2]
    rng = np.random.default_rng(5)
    zt = rng.standard_normal((13, 2))
    m = oracle.reduce_mean(lengths, zt)
    o = [0, 9]
    eta = [0, 3]
    for i, n in enumerate(lengths):
        for a in range(n):
            acc = [0.0, 0.0]
            for b in range(n):
                for f in range(2):
                    acc[f] += zt[o[i] + a * n + b, f]
            for f in range(2):
                assert abs(m[eta[i] + a, f] - acc[f] / n) < 1e-14


# -------------------------------------------------------------- invariances
def test_sample_permutation_permutes_outputs():
    lengths = [5, 2, 7, 3]
    x = pin.make_inputs(lengths, 16, 8, 16, "f32", seed=8)
    w = _w64(x.weights[0])
    so, zo = oracle.block(lengths, x.s.f64, w)
    perm = [2, 0, 3, 1]
    eta = np.concatenate([[0], np.cumsum(lengths)])
    o = np.concatenate([[0], np.cumsum(np.square(lengths))])
    s_p = np.concatenate([x.s.f64[eta[i]:eta[i + 1]] for i in perm])
    so_p, zo_p = oracle.block([lengths[i] for i in perm], s_p, w)
    np.testing.assert_allclose(so_p, np.concatenate([so[eta[i]:eta[i + 1]] for i in perm]),
                               rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(zo_p, np.concatenate([zo[o[i]:o[i + 1]] for i in perm]),
                               rtol=1e-14, atol=1e-14)


def test_batch_split_concatenates():
    lengths = [4, 6, 1, 3]
    x = pin.make_inputs(lengths, 16, 8, 16, "f32", seed=9)
    w = _w64(x.weights[0])
    so, zo = oracle.block(lengths, x.s.f64, w)
    sa, za = oracle.block(lengths[:2], x.s.f64[:10], w)
    sb, zb = oracle.block(lengths[2:], x.s.f64[10:], w)
    np.testing.assert_allclose(so, np.concatenate([sa, sb]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(zo, np.concatenate([za, zb]), rtol=1e-14, atol=1e-14)


def test_chain_composes_blocks():
    lengths = [3, 5]
    x = pin.make_inputs(lengths, 16, 8, 16, "f32", blocks=2, seed=10)
    ws = [_w64(w) for w in x.weights]
    s1, _ = oracle.block(lengths, x.s.f64, ws[0])
    s2, z2 = oracle.block(lengths, s1, ws[1])
    sc, zc = oracle.chain(lengths, x.s.f64, ws)
    assert (sc == s2).all() and (zc == z2).all()
    s_one, z_one = oracle.chain(lengths, x.s.f64, ws[:1])
    assert (s_one == s1).all()


def test_sampled_forms_match_full_block():
    lengths = [9, 0, 14, 5]
    x = pin.make_inputs(lengths, 32, 16, 32, "bf16", seed=12)
    w = _w64(x.weights[0])
    so, zo = oracle.block(lengths, x.s.f64, w)
    cells = np.array([0, 5, 80, 81, 276, len(zo) - 1])
    np.testing.assert_allclose(oracle.block_cells(lengths, x.s.f64, w, cells), zo[cells],
                               rtol=1e-13, atol=1e-13)
    a = oracle.project(x.s.f64, w["Wa"])
    b = oracle.project(x.s.f64, w["Wb"])
    np.testing.assert_array_equal(oracle.broadcast_cells(lengths, a, b, cells),
                                  oracle.broadcast(lengths, a, b)[cells])
    rows = np.array([0, 8, 9, 22, 27])
    m_full = oracle.reduce_mean(lengths, zo)
    m_r, s_r = oracle.block_rows(lengths, x.s.f64, w, rows)
    np.testing.assert_allclose(m_r, m_full[rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s_r, so[rows], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------ exact inputs
def test_exact_inputs_stay_integral():
    lengths = [2, 4, 8, 16]
    for dtype in ("f32", "bf16"):
        x = pin.exact_inputs(lengths, 16, 16, 32, dtype, seed=1)
        w = _w64(x.weights[0])
        s = x.s.f64
        a, b = oracle.project(s, w["Wa"]), oracle.project(s, w["Wb"])
        z = oracle.broadcast(lengths, a, b)
        zt = oracle.transition(z, w["W1"], w["W2"])
        m = oracle.reduce_mean(lengths, zt)
        for v in (a, b, z, zt):
            assert (v == np.round(v)).all() and np.abs(v).max() <= 256
        Nrow = np.repeat(lengths, lengths)[:, None]
        assert (m * Nrow == np.round(m * Nrow)).all()


# ------------------------------------------------------------ bf16 rounding
def test_round_bf16_ties_and_double_rounding():
    one = 1.0
    cases = {
        one + 2.0 ** -8: one,                            # tie -> even (down)
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,            # tie -> even (up)
        one + 2.0 ** -8 + 2.0 ** -40: one + 2.0 ** -7,   # above tie (fp32 first would tie)
        -(one + 2.0 ** -8 + 2.0 ** -40): -(one + 2.0 ** -7),
        3.0: 3.0,
        1.0 / 3.0: 0.333984375,
    }
    for x, want in cases.items():
        assert oracle.round_bf16(np.array([x]))[0] == want, x


def test_round_bf16_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (oracle.bf16_bits(x32.astype(np.float64)) == ref).all()


# ------------------------------------------- pre-normalised SwiGLU transition
def test_layer_norm_hand_computed():
    # row [2, 2, 2, 6]: mean 3, biased variance (1 + 1 + 1 + 9) / 4 = 3
    z = np.array([[1.0, 3.0]])
    got = oracle.layer_norm(z, [1.0, 1.0], [0.0, 0.0], 0.0)
    assert np.allclose(got[0], [-1.0, 1.0], rtol=0, atol=1e-15)
    got = oracle.layer_norm([[2.0, 2.0, 2.0, 6.0]], [2.0, 1.0, 1.0, 1.0], [0.0, 0.0, 0.0, 5.0], 0.0)
    r3 = np.sqrt(3.0)
    assert np.allclose(got[0], [-2 / r3, -1 / r3, -1 / r3, 3 / r3 + 5.0], rtol=0, atol=1e-14)
    # eps enters under the square root: var 3 + eps 1 -> divide by 2
    got = oracle.layer_norm([[2.0, 2.0, 2.0, 6.0]], np.ones(4), np.zeros(4), 1.0)
    assert np.allclose(got[0], [-0.5, -0.5, -0.5, 1.5], rtol=0, atol=1e-15)


def test_layer_norm_invariances():
    rng = np.random.default_rng(40)
    z = rng.standard_normal((30, 16))
    g, b = np.ones(16), np.zeros(16)
    x = oracle.layer_norm(z, g, b, 0.0)
    assert np.allclose(x.mean(axis=1), 0.0, atol=1e-13)
    assert np.allclose(np.square(x).mean(axis=1), 1.0, atol=1e-12)
    shift = rng.standard_normal((30, 1)) * 10
    assert np.allclose(oracle.layer_norm(z + shift, g, b, 0.0), x, atol=1e-12)
    scale = rng.uniform(0.1, 10.0, (30, 1))
    assert np.allclose(oracle.layer_norm(z * scale, g, b, 0.0), x, atol=1e-12)


def test_layer_norm_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    z = rng.standard_normal((50, 24)) * 3 + 1
    g, b = rng.standard_normal(24), rng.standard_normal(24)
    want = torch.nn.functional.layer_norm(torch.from_numpy(z), (24,), torch.from_numpy(g),
                                          torch.from_numpy(b), eps=1e-5).numpy()
    assert np.allclose(oracle.layer_norm(z, g, b, 1e-5), want, rtol=1e-12, atol=1e-12)


def test_swiglu_zero_weights_is_identity():
    rng = np.random.default_rng(42)
    z = rng.standard_normal((20, 8))
    g, b = rng.standard_normal(8), rng.standard_normal(8)
    Wg, Wu, Wd = (rng.standard_normal(s) for s in ((16, 8), (16, 8), (8, 16)))
    for args in ((np.zeros_like(Wg), Wu, Wd), (Wg, np.zeros_like(Wu), Wd),
                 (Wg, Wu, np.zeros_like(Wd))):
        assert (oracle.transition_swiglu(z, g, b, *args) == z).all()


def test_swiglu_hand_computed():
    # z = [1, 3], eps = 0 -> x = [-1, 1]; g = -0.5 + 1.5 = 1; u = -2 + 1 = -1;
    # silu(1) = 1 / (1 + e^-1); update = silu(1) * u * [1, -2]
    s1 = 1.0 / (1.0 + np.exp(-1.0))
    got = oracle.transition_swiglu([[1.0, 3.0]], [1.0, 1.0], [0.0, 0.0], [[0.5, 1.5]],
                                   [[2.0, 1.0]], [[1.0], [-2.0]], eps=0.0)
    assert np.allclose(got[0], [1.0 - s1, 3.0 + 2.0 * s1], rtol=0, atol=1e-14)
    # gate and value are not interchangeable: swapping Wg and Wu changes the result
    swapped = oracle.transition_swiglu([[1.0, 3.0]], [1.0, 1.0], [0.0, 0.0], [[2.0, 1.0]],
                                       [[0.5, 1.5]], [[1.0], [-2.0]], eps=0.0)
    sm1 = -1.0 / (1.0 + np.exp(1.0))          # silu(-1)
    assert np.allclose(swapped[0], [1.0 + sm1 * 1.0, 3.0 - 2.0 * sm1], rtol=0, atol=1e-14)


def test_swiglu_matches_torch():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(43)
    z = rng.standard_normal((64, 16))
    g, b = rng.standard_normal(16), rng.standard_normal(16)
    Wg, Wu = rng.standard_normal((48, 16)) / 4, rng.standard_normal((48, 16)) / 4
    Wd = rng.standard_normal((16, 48)) / 7
    t = lambda a: torch.from_numpy(np.asarray(a))
    x = F.layer_norm(t(z), (16,), t(g), t(b), eps=1e-5)
    want = (t(z) + F.linear(F.silu(F.linear(x, t(Wg))) * F.linear(x, t(Wu)), t(Wd))).numpy()
    assert np.allclose(oracle.transition_swiglu(z, g, b, Wg, Wu, Wd), want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ rectangular pairs
def test_rect_partition_hand_computed():
    # N = [2, 0, 3], M = [4, 5, 1]: sample 0 is 2 x 4 (cells 0..7, rows at 0, 4),
    # sample 1 has no rows (and no cells, although M_1 = 5), sample 2 is 3 x 1
    # (cells 8, 9, 10, one per row).
    p = oracle.partition_rect([2, 0, 3], [4, 5, 1])
    assert p["T"] == 5 and p["T_cols"] == 10 and p["cells"] == 11
    assert p["single_offsets"].tolist() == [0, 2, 2, 5]
    assert p["col_offsets"].tolist() == [0, 4, 9, 10]
    assert p["pair_offsets"].tolist() == [0, 8, 8, 11]
    assert p["row_splits"].tolist() == [0, 4, 8, 9, 10, 11]
    assert p["row_sample"].tolist() == [0, 0, 2, 2, 2]
    sample, row, col = oracle.decode_cells_rect([2, 0, 3], [4, 5, 1])
    assert sample.tolist() == [0] * 8 + [2] * 3
    assert row.tolist() == [0, 0, 0, 0, 1, 1, 1, 1, 0, 1, 2]
    assert col.tolist() == [0, 1, 2, 3, 0, 1, 2, 3, 0, 0, 0]


@pytest.mark.parametrize("lengths", [[7, 12, 5, 16], [0, 3, 0, 1, 17, 0], [9]])
def test_rect_with_equal_axes_is_square(lengths):
    rng = np.random.default_rng(60)
    p, q = oracle.partition_rect(lengths, lengths), oracle.partition(lengths)
    for k in ("single_offsets", "pair_offsets", "row_splits", "row_sample"):
        assert (p[k] == q[k]).all(), k
    assert (p["col_offsets"] == q["single_offsets"]).all()
    for u, v in zip(oracle.decode_cells_rect(lengths, lengths), oracle.decode_cells(lengths)):
        assert (u == v).all()
    T = sum(lengths)
    a, b = rng.standard_normal((T, 6)), rng.standard_normal((T, 6))
    z = oracle.broadcast_rect(lengths, lengths, a, b)
    assert (z == oracle.broadcast(lengths, a, b)).all()
    assert (oracle.reduce_mean_rect(lengths, lengths, z) == oracle.reduce_mean(lengths, z)).all()


def test_rect_broadcast_bruteforce():
    rows, cols = [3, 1, 0, 2], [2, 4, 3, 5]
    rng = np.random.default_rng(61)
    a = rng.standard_normal((sum(rows), 3))
    b = rng.standard_normal((sum(cols), 3))
    z = oracle.broadcast_rect(rows, cols, a, b)
    t = eta = mu = 0
    for n, m in zip(rows, cols):
        for r in range(n):
            for c in range(m):
                for f in range(3):
                    assert z[t, f] == a[eta + r, f] + b[mu + c, f]
                t += 1
        eta, mu = eta + n, mu + m
    assert t == z.shape[0]


def test_rect_reduce_closed_form_without_transition():
    # no transition: mean_c (a[eta + r] + b[mu + c]) = a[eta + r] + mean(b of the sample)
    rows, cols = [4, 2, 3], [3, 7, 1]
    rng = np.random.default_rng(62)
    a = rng.standard_normal((sum(rows), 5))
    b = rng.standard_normal((sum(cols), 5))
    m = oracle.reduce_mean_rect(rows, cols, oracle.broadcast_rect(rows, cols, a, b))
    eta = np.concatenate([[0], np.cumsum(rows)])
    mu = np.concatenate([[0], np.cumsum(cols)])
    want = np.concatenate([a[eta[i]:eta[i + 1]] + b[mu[i]:mu[i + 1]].mean(axis=0)
                           for i in range(3)])
    assert np.allclose(m, want, rtol=0, atol=1e-14)


def test_rect_block_equals_dense_per_sample():
    rows, cols = [5, 0, 3, 8], [2, 6, 9, 1]
    rng = np.random.default_rng(63)
    c_s, c_z, h = 6, 4, 8
    w = {"Wa": rng.standard_normal((c_z, c_s)), "Wb": rng.standard_normal((c_z, c_s)),
         "W1": rng.standard_normal((h, c_z)), "W2": rng.standard_normal((c_z, h)),
         "Wo": rng.standard_normal((c_s, c_z))}
    s_rows = rng.standard_normal((sum(rows), c_s))
    s_cols = rng.standard_normal((sum(cols), c_s))
    s_new, zt = oracle.block_rect(rows, cols, s_rows, s_cols, w)
    eta = np.concatenate([[0], np.cumsum(rows)])
    mu = np.concatenate([[0], np.cumsum(cols)])
    o = np.concatenate([[0], np.cumsum(np.multiply(rows, cols))])
    for i in range(len(rows)):
        X, Y = s_rows[eta[i]:eta[i + 1]], s_cols[mu[i]:mu[i + 1]]
        P = (X @ w["Wa"].T)[:, None, :] + (Y @ w["Wb"].T)[None, :, :]   # [N, M, c_z]
        Pt = P + np.maximum(P @ w["W1"].T, 0.0) @ w["W2"].T
        assert np.allclose(zt[o[i]:o[i + 1]], Pt.reshape(-1, c_z), rtol=1e-12, atol=1e-12)
        if rows[i] and cols[i]:
            want = X + Pt.mean(axis=1) @ w["Wo"].T
            assert np.allclose(s_new[eta[i]:eta[i + 1]], want, rtol=1e-12, atol=1e-12)


def test_swiglu_block_closed_form_and_dense():
    """The SwiGLU block: with Wd = 0 the transition is the identity and the
    column mean is a + mean_c b (as for the ReLU block with W2 = 0); for any
    weights each sample equals the dense per-sample formula (the transition
    applied to the outer sum, a mean over axis 1)."""
    rng = np.random.default_rng(31)
    lengths, c_s, c_z, hidden = [3, 0, 5, 2], 6, 4, 8
    s = rng.normal(size=(sum(lengths), c_s))
    w = {"Wa": rng.normal(size=(c_z, c_s)), "Wb": rng.normal(size=(c_z, c_s)),
         "Wo": rng.normal(size=(c_s, c_z)), "ln_gamma": 1 + rng.normal(size=c_z),
         "ln_beta": rng.normal(size=c_z), "Wg": rng.normal(size=(hidden, c_z)),
         "Wu": rng.normal(size=(hidden, c_z)), "Wd": np.zeros((c_z, hidden))}
    s_out, z_out = oracle.block_swiglu(lengths, s, w)
    a, b = s @ w["Wa"].T, s @ w["Wb"].T
    eta = np.concatenate([[0], np.cumsum(lengths)])
    m = np.concatenate([a[eta[i]:eta[i + 1]] + b[eta[i]:eta[i + 1]].mean(axis=0)
                        for i in range(len(lengths)) if lengths[i]])
    np.testing.assert_allclose(s_out, s + m @ w["Wo"].T, rtol=1e-12, atol=1e-12)
    w["Wd"] = rng.normal(size=(c_z, hidden))
    s_out, z_out = oracle.block_swiglu(lengths, s, w)
    o = 0
    for i, n in enumerate(lengths):
        X = s[eta[i]:eta[i + 1]]
        P = (X @ w["Wa"].T)[:, None, :] + (X @ w["Wb"].T)[None, :, :]
        Pt = oracle.transition_swiglu(P.reshape(-1, c_z), w["ln_gamma"], w["ln_beta"], w["Wg"],
                                      w["Wu"], w["Wd"]).reshape(n, n, c_z)
        np.testing.assert_allclose(z_out[o:o + n * n], Pt.reshape(-1, c_z), rtol=1e-12)
        if n:
            np.testing.assert_allclose(s_out[eta[i]:eta[i + 1]],
                                       X + Pt.mean(axis=1) @ w["Wo"].T, rtol=1e-12)
        o += n * n
