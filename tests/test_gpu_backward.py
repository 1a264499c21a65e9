"""GPU parity of the backward pass and Equation 5's loss against the oracle
(fp32: 1e-5; bf16: 2e-2, scaled max error), through the C ABI.

The relu mask is a decision taken in floating point: the oracle takes it on
the exact pair state, the kernels on their stored operand (bf16 z in bf16)
with fp32 sums, and a unit whose exact pre-activation lies within that
error of zero may fall on either side, moving the gradient by its whole
term. relu_kinks bounds those units from the oracle's values, fits the flips
that explain one observable output (g_z per cell, or dW1 per unit), carries
them through the later, linear adjoints and then compares every element of
every output with the tolerance: no cell is filtered and the reference is
the plain float64 oracle. Exact inputs (integer singles, sparse +-1
weights, power-of-two lengths, small-integer incoming gradients) check the
same paths with every decision and operand exact on both sides."""
import numpy as np
import pytest

import oracle
import pair_inputs as pin
from gpu_util import announce, f64, to_dev, weights_to_dev
from helpers import TOL, scaled_max_err
import relu_kinks

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def nt():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import padding_free_pair_amd as nt
    nt._native.lib()  # raises if the library is missing: no fallback
    return nt


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("name,rows,cols,c_s,c_z,dtype", [
    ("tiny", [7, 12, 5, 16], None, 16, 8, "f32"),
    ("bf16", [9, 40, 2, 0, 33], None, 128, 64, "bf16"),
    ("rect", [3, 0, 5, 2], [4, 2, 1, 6], 16, 24, "bf16"),
    ("long_rows", [300, 2], [1, 400], 8, 16, "f32"),
])
def test_loss_eq5(nt, name, rows, cols, c_s, c_z, dtype):
    announce(f"loss eq5 {name}")
    cols_ = rows if cols is None else cols
    cells = int(np.dot(rows, cols_))
    x = pin.random_rows(sum(rows), c_s, dtype, seed=1)
    pz = pin.random_rows(cells, c_z, dtype, seed=2)
    p = nt.nt_make_partition(rows) if cols is None else nt.nt_make_partition_rect(rows, cols)
    for S in (1, 3):
        # S > 1: rows of S slices (the non-leading layout); slices differ
        xs = pin.random_rows(sum(rows), S * c_s, dtype, seed=1) if S > 1 else x
        ps = pin.random_rows(cells, S * c_z, dtype, seed=2) if S > 1 else pz
        loss, gx, gp = nt.nt_pair_loss_eq5(p, to_dev(xs, torch), to_dev(ps, torch), S=S)
        torch.cuda.synchronize()
        L, rgx, rgp = oracle.loss_eq5(rows, cols_, xs.f64, ps.f64, S=S)
        assert float(loss.cpu()[0]) == pytest.approx(L, rel=1e-5)
        assert scaled_max_err(gx.cpu().numpy(), rgx) <= 1e-6
        assert scaled_max_err(gp.cpu().numpy(), rgp) <= 1e-6


def test_loss_eq5_empty_samples(nt):
    announce("loss eq5 empty")
    p = nt.nt_make_partition([0, 0])
    x = torch.empty((0, 8), device="cuda")
    pz = torch.empty((0, 8), device="cuda")
    loss, gx, gp = nt.nt_pair_loss_eq5(p, x, pz)
    torch.cuda.synchronize()
    assert float(loss.cpu()[0]) == 0.0


@pytest.mark.parametrize("rows,cols,c_z", [
    ([7, 12, 5, 16], None, 128),
    ([3, 0, 5, 2], [4, 2, 1, 6], 24),
    ([300, 2], [1, 400], 64),
    ([1] * 300, None, 8),
])
def test_mean_and_broadcast_adjoints(nt, rows, cols, c_z):
    announce(f"mean/broadcast adjoints B={len(rows)} c_z={c_z}")
    cols_ = rows if cols is None else cols
    cells = int(np.dot(rows, cols_))
    rng = np.random.default_rng(5)
    gm = rng.standard_normal((sum(rows), c_z)).astype(np.float32)
    gin = rng.standard_normal((cells, c_z)).astype(np.float32)
    p = nt.nt_make_partition(rows) if cols is None else nt.nt_make_partition_rect(rows, cols)
    G = nt.nt_pair_reduce_backward(p, _f32(gm), _f32(gin))
    G0 = nt.nt_pair_reduce_backward(p, _f32(gm))
    gz = _f32(gin)
    nt.nt_pair_reduce_backward(p, _f32(gm), gz, G=gz)  # in place
    g_a, g_b = nt.nt_pair_broadcast_backward(p, _f32(gin))
    torch.cuda.synchronize()
    ref = oracle.reduce_mean_backward(rows, cols_, gm.astype(np.float64))
    assert scaled_max_err(G0.cpu().numpy(), ref) <= 1e-6
    assert scaled_max_err(G.cpu().numpy(), ref + gin) <= 1e-6
    np.testing.assert_array_equal(gz.cpu().numpy(), G.cpu().numpy())
    ra, rb = oracle.broadcast_backward(rows, cols_, gin.astype(np.float64))
    assert scaled_max_err(g_a.cpu().numpy(), ra) <= 1e-5
    assert scaled_max_err(g_b.cpu().numpy(), rb) <= 1e-5


@pytest.mark.parametrize("lengths,c_z,hidden,dtype", [
    ([7, 12, 5, 16], 8, 16, "f32"),
    ([7, 12, 5, 16], 48, 40, "bf16"),
    ([9, 40, 2, 33], 128, 512, "bf16"),    # matrix-core kernels, ragged last tile
    ([1], 128, 512, "bf16"),               # one cell
    ([33, 100, 7, 0, 61], 128, 512, "bf16"),  # many tiles and split-K slices
    ([16, 3, 1], 64, 128, "bf16"),
])
def test_transition_backward(nt, lengths, c_z, hidden, dtype):
    announce(f"transition backward c_z={c_z} hidden={hidden} {dtype}")
    cells = int(np.square(lengths).sum())
    z = pin.random_rows(cells, c_z, dtype, seed=11)
    G = np.random.default_rng(12).standard_normal((cells, c_z)).astype(np.float32)
    W1 = pin.random_rows(hidden, c_z, dtype, seed=13, scale=1 / np.sqrt(c_z))
    W2 = pin.random_rows(c_z, hidden, dtype, seed=14, scale=1 / np.sqrt(hidden))
    p = nt.nt_make_partition(lengths)
    g_z, dW1, dW2 = nt.nt_pair_transition_backward(p, to_dev(z, torch), _f32(G),
                                                   to_dev(W1, torch), to_dev(W2, torch))
    Gd = _f32(G)
    g_z2, _, _ = nt.nt_pair_transition_backward(p, to_dev(z, torch), Gd, to_dev(W1, torch),
                                                to_dev(W2, torch), g_z=Gd)  # in place
    torch.cuda.synchronize()
    rz, r1, r2, nf, nc = relu_kinks.transition_reference(z.f64, W1.f64, W2.f64,
                                                         G.astype(np.float64), g_z.cpu().numpy())
    announce(f"relu flips fitted {nf} of {nc} candidates")
    tol = TOL[dtype]
    assert scaled_max_err(g_z.cpu().numpy(), rz) <= tol
    assert scaled_max_err(dW1.cpu().numpy(), r1) <= tol
    assert scaled_max_err(dW2.cpu().numpy(), r2) <= tol
    np.testing.assert_array_equal(g_z2.cpu().numpy(), g_z.cpu().numpy())


def test_transition_backward_full_size(nt):
    """The high-variation workload's cells (bf16, c_z 128, hidden 512) in the
    benchmark's launch configuration: g_z on every cell, dW1 and dW2."""
    x = pin.workload_inputs(3, blocks=1)
    lengths = x.lengths.tolist()
    cells = int(np.square(x.lengths.astype(np.int64)).sum())
    announce(f"transition backward full size cells={cells}")
    z = pin.random_rows(cells, 128, "bf16", seed=41)
    G = (np.random.default_rng(42).standard_normal((cells, 128)) / 64).astype(np.float32)
    W1, W2 = x.weights[0]["W1"], x.weights[0]["W2"]
    p = nt.nt_make_partition(lengths)
    g_z, dW1, dW2 = nt.nt_pair_transition_backward(p, to_dev(z, torch), _f32(G),
                                                   to_dev(W1, torch), to_dev(W2, torch))
    torch.cuda.synchronize()
    got = g_z.cpu().numpy()
    rz, r1, r2, nf, nc = relu_kinks.transition_reference(z.f64, W1.f64, W2.f64,
                                                         G.astype(np.float64), got)
    announce(f"relu flips fitted {nf} of {nc} candidates")
    assert scaled_max_err(got, rz) <= TOL["bf16"]
    assert scaled_max_err(dW1.cpu().numpy(), r1) <= TOL["bf16"]
    assert scaled_max_err(dW2.cpu().numpy(), r2) <= TOL["bf16"]


@pytest.mark.parametrize("lengths,c_s,c_z,hidden,dtype,with_gz,inputs", [
    ([7, 12, 5, 16], 16, 8, 16, "f32", True, "random"),
    ([7, 12, 5, 16], 16, 8, 16, "f32", False, "random"),
    ([9, 20, 2, 0, 13], 128, 64, 128, "bf16", True, "random"),
    ([8, 16, 4], 64, 128, 512, "bf16", True, "exact"),
    ([8, 16, 4], 64, 128, 512, "bf16", False, "exact"),
    ([9, 20, 13], 64, 128, 512, "bf16", True, "random"),     # the pages' widths
    ([9, 20, 13], 64, 128, 512, "bf16", False, "random"),
    ([6, 11, 0, 9], 384, 128, 512, "bf16", True, "random"),   # the four-block widths
])
def test_block_backward(nt, lengths, c_s, c_z, hidden, dtype, with_gz, inputs):
    announce(f"block backward c_s={c_s} c_z={c_z} hidden={hidden} {dtype} gz={with_gz} {inputs}")
    if inputs == "exact":
        x = pin.exact_inputs(lengths, c_s, c_z, hidden, dtype, seed=21)
    else:
        x = pin.make_inputs(lengths, c_s, c_z, hidden, dtype, seed=21)
    w = x.weights[0]
    cells = int(np.square(lengths).sum())
    rng = np.random.default_rng(22)
    if inputs == "exact":
        gs = rng.integers(-2, 3, (sum(lengths), c_s)).astype(np.float32)
        gz = rng.integers(-2, 3, (cells, c_z)).astype(np.float32) if with_gz else None
    else:
        gs = rng.standard_normal((sum(lengths), c_s)).astype(np.float32)
        gz = rng.standard_normal((cells, c_z)).astype(np.float32) if with_gz else None
    p = nt.nt_make_partition(lengths)
    wd = weights_to_dev(w, torch)
    sd = to_dev(x.s, torch)
    s_out, z_out = nt.nt_pair_block(p, sd, wd)
    g_s, grads = nt.nt_pair_block_backward(p, sd, z_out, wd, _f32(gs),
                                           None if gz is None else _f32(gz))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in grads.items()}
    W64 = {k: v.f64 for k, v in w.items()}
    gz64 = None if gz is None else gz.astype(np.float64)
    if inputs == "exact":
        # every operand and pre-activation is exact on both sides: the plain
        # oracle, relu decisions included
        ref = oracle.block_backward(lengths, x.s.f64, W64, gs.astype(np.float64), gz64)
    else:
        ref, nf, nc = relu_kinks.block_reference(lengths, x.s.f64, W64, gs.astype(np.float64),
                                                 gz64, got["W1"], dtype == "bf16")
        announce(f"relu flips fitted {nf} of {nc} candidates")
    tol = TOL[dtype]
    assert scaled_max_err(g_s.cpu().numpy(), ref["s"]) <= tol
    for k in ("Wa", "Wb", "W1", "W2", "Wo"):
        assert scaled_max_err(got[k], ref[k]) <= tol, k


def test_chain_backward_under_eq5(nt):
    """Two blocks and Equation 5 end to end (fp32): loss, single gradient and
    every weight gradient against the oracle's chain."""
    announce("chain backward fp32")
    lengths = [7, 12, 5, 16]
    x = pin.make_inputs(lengths, 16, 8, 16, "f32", blocks=2, seed=31)
    p = nt.nt_make_partition(lengths)
    ws = [weights_to_dev(w, torch) for w in x.weights]
    s = [to_dev(x.s, torch)]
    zs = []
    for w in ws:
        so, zo = nt.nt_pair_block(p, s[-1], w)
        s.append(so)
        zs.append(zo)
    loss, g_x, g_pz = nt.nt_pair_loss_eq5(p, s[-1], zs[-1])
    g = g_x
    grads = [None, None]
    for k in (1, 0):
        g, grads[k] = nt.nt_pair_block_backward(p, s[k], zs[k], ws[k], g,
                                                g_pz if k == 1 else None)
    torch.cuda.synchronize()
    L, rg, rgrads = oracle.chain_backward(lengths, x.s.f64,
                                          [{k: v.f64 for k, v in w.items()} for w in x.weights])
    assert float(loss.cpu()[0]) == pytest.approx(L, rel=1e-5)
    assert scaled_max_err(g.cpu().numpy(), rg) <= TOL["f32"]
    for k in range(2):
        for name in rgrads[k]:
            assert scaled_max_err(grads[k][name].cpu().numpy(), rgrads[k][name]) <= TOL["f32"]


@pytest.mark.parametrize("lengths", [[0, 0, 0], [0]])
def test_block_backward_empty_batch(nt, lengths):
    """No singles and no cells: every gradient is zero, nothing is read."""
    announce(f"block backward empty {lengths}")
    c_s, c_z, hidden = 64, 128, 512
    x = pin.make_inputs([1], c_s, c_z, hidden, "bf16", seed=3)   # weights only
    p = nt.nt_make_partition(lengths)
    wd = weights_to_dev(x.weights[0], torch)
    s = torch.empty((0, c_s), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((0, c_z), dtype=torch.bfloat16, device="cuda")
    gs = torch.empty((0, c_s), dtype=torch.float32, device="cuda")
    g, grads = nt.nt_pair_block_backward(p, s, z, wd, gs)
    torch.cuda.synchronize()
    assert g.numel() == 0
    for k, v in grads.items():
        assert torch.count_nonzero(v).item() == 0, k


def test_block_backward_many_samples(nt):
    """More samples than the one-launch partition takes (B = 300), with
    empty samples among them, fp32 against the oracle."""
    rng = np.random.default_rng(17)
    lengths = rng.integers(0, 6, 300).tolist()
    announce(f"block backward B={len(lengths)} T={sum(lengths)}")
    x = pin.make_inputs(lengths, 16, 8, 16, "f32", seed=18)
    w = x.weights[0]
    cells = int(np.square(lengths).sum())
    gs = rng.standard_normal((sum(lengths), 16)).astype(np.float32)
    gz = rng.standard_normal((cells, 8)).astype(np.float32)
    p = nt.nt_make_partition(lengths)
    wd = weights_to_dev(w, torch)
    sd = to_dev(x.s, torch)
    _, z_out = nt.nt_pair_block(p, sd, wd)
    g, grads = nt.nt_pair_block_backward(p, sd, z_out, wd, _f32(gs), _f32(gz))
    torch.cuda.synchronize()
    ref = oracle.block_backward(lengths, x.s.f64, {k: v.f64 for k, v in w.items()},
                                gs.astype(np.float64), gz.astype(np.float64))
    assert scaled_max_err(g.cpu().numpy(), ref["s"]) <= TOL["f32"]
    for k in ("Wa", "Wb", "W1", "W2", "Wo"):
        assert scaled_max_err(grads[k].cpu().numpy(), ref[k]) <= TOL["f32"], k


def test_transition_backward_no_cells(nt):
    announce("transition backward, no cells")
    p = nt.nt_make_partition([0, 0])
    z = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    G = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    W1 = torch.ones((512, 128), dtype=torch.bfloat16, device="cuda")
    W2 = torch.ones((128, 512), dtype=torch.bfloat16, device="cuda")
    dW1 = torch.full((512, 128), 7.0, device="cuda")
    dW2 = torch.full((128, 512), 7.0, device="cuda")
    nt.nt_pair_transition_backward(p, z, G, W1, W2, dW1=dW1, dW2=dW2)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW1).item() == 0 and torch.count_nonzero(dW2).item() == 0
