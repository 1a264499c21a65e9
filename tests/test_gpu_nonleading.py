"""GPU parity of the non-leading (S, N_i, C) layout (Appendix A.1's
non-leading variant, S = 3): the block and its gradients through the C ABI
against the oracle (fp32: 1e-5; bf16: 2e-2). bf16 gradients on random
inputs carry the relu flips fitted within the operand's error window
(relu_kinks, as in test_gpu_backward.py); exact inputs make every decision
and operand exact on both sides."""
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


def _inputs(lengths, S, c_s, c_z, hidden, dtype, exact, seed):
    if exact:
        x = pin.exact_inputs(lengths, S * c_s, c_z, hidden, dtype, seed=seed)
        # exact_inputs draws Wa, Wb over S * c_s inputs; redraw them at c_s
        ex = pin.exact_inputs(lengths, c_s, c_z, hidden, dtype, seed=seed + 1)
        return x.s, ex.weights[0]
    x = pin.make_inputs(lengths, c_s, c_z, hidden, dtype, seed=seed)
    s = pin.random_rows(int(sum(lengths)), S * c_s, dtype, seed=seed + 7)
    return s, x.weights[0]


@pytest.mark.parametrize("lengths,S,c_s,c_z,hidden,dtype", [
    ([7, 12, 5, 16], 3, 16, 8, 16, "f32"),
    ([7, 12, 0, 5, 16], 3, 64, 128, 512, "bf16"),   # the pages' widths: S * c_z = 384
    ([9, 20, 13], 2, 32, 64, 128, "bf16"),
])
def test_block_nl_forward(nt, lengths, S, c_s, c_z, hidden, dtype):
    announce(f"non-leading block S={S} c_z={c_z} hidden={hidden} {dtype}")
    s, w = _inputs(lengths, S, c_s, c_z, hidden, dtype, False, 3)
    p = nt.nt_make_partition(lengths)
    so, zo = nt.nt_pair_block_nl(p, to_dev(s, torch), weights_to_dev(w, torch), S)
    torch.cuda.synchronize()
    rs, rz = oracle.block_nl(lengths, s.f64, {k: v.f64 for k, v in w.items()}, S)
    assert scaled_max_err(f64(zo, torch), rz) <= TOL[dtype]
    assert scaled_max_err(f64(so, torch), rs) <= TOL[dtype]


@pytest.mark.parametrize("lengths,S,c_s,c_z,hidden,dtype,exact", [
    ([7, 12, 5, 16], 3, 16, 8, 16, "f32", False),
    ([8, 16, 4], 3, 64, 128, 512, "bf16", True),
    ([8, 4, 0, 2], 2, 32, 64, 128, "bf16", True),
    ([9, 20, 0, 13], 3, 64, 128, 512, "bf16", False),   # the pages' widths, random inputs
])
def test_block_nl_backward(nt, lengths, S, c_s, c_z, hidden, dtype, exact):
    announce(f"non-leading backward S={S} c_z={c_z} hidden={hidden} {dtype}")
    s, w = _inputs(lengths, S, c_s, c_z, hidden, dtype, exact, 5)
    cells = int(np.square(lengths).sum())
    rng = np.random.default_rng(6)
    if exact:
        gs = rng.integers(-2, 3, (sum(lengths), S * c_s)).astype(np.float32)
        gz = rng.integers(-2, 3, (cells, S * c_z)).astype(np.float32)
    else:
        gs = rng.standard_normal((sum(lengths), S * c_s)).astype(np.float32)
        gz = rng.standard_normal((cells, S * c_z)).astype(np.float32)
    p = nt.nt_make_partition(lengths)
    wd = weights_to_dev(w, torch)
    sd = to_dev(s, torch)
    so, zo = nt.nt_pair_block_nl(p, sd, wd, S)
    g, grads = nt.nt_pair_block_backward_nl(p, sd, zo, wd, S, _f32(gs), _f32(gz))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in grads.items()}
    W64 = {k: v.f64 for k, v in w.items()}
    if exact:
        # every operand and pre-activation is exact on both sides
        ref = oracle.block_backward_nl(lengths, s.f64, W64, S, gs.astype(np.float64),
                                       gz.astype(np.float64))
    else:
        ref, nf, nc = relu_kinks.block_reference(lengths, s.f64, W64, gs.astype(np.float64),
                                                 gz.astype(np.float64), got["W1"],
                                                 dtype == "bf16", S=S)
        announce(f"relu flips fitted {nf} of {nc} candidates")
    tol = TOL[dtype]
    assert scaled_max_err(g.cpu().numpy(), ref["s"]) <= tol
    for k in ("Wa", "Wb", "W1", "W2", "Wo"):
        assert scaled_max_err(got[k], ref[k]) <= tol, k


def test_nl_with_one_slice_is_the_leading_block(nt):
    lengths = [7, 12, 5, 16, 33]
    announce("non-leading S = 1 against the leading block")
    x = pin.workload_inputs(1, blocks=1)
    p = nt.nt_make_partition(lengths)
    s = pin.random_rows(sum(lengths), x.c_s, x.dtype, seed=5)
    w = weights_to_dev(x.weights[0], torch)
    sd = to_dev(s, torch)
    s_a, z_a = nt.nt_pair_block(p, sd, w)
    s_b, z_b = nt.nt_pair_block_nl(p, sd, w, 1)
    torch.cuda.synchronize()
    assert torch.equal(s_a, s_b) and torch.equal(z_a, z_b)


def test_block_nl_many_samples(nt):
    """B = 300 (two-launch partition), S = 3, fp32: forward and backward."""
    rng = np.random.default_rng(21)
    lengths = rng.integers(0, 6, 300).tolist()
    S, c_s, c_z, hidden = 3, 8, 8, 16
    announce(f"non-leading B={len(lengths)} S={S}")
    s, w = _inputs(lengths, S, c_s, c_z, hidden, "f32", False, 22)
    cells = int(np.square(lengths).sum())
    gs = rng.standard_normal((sum(lengths), S * c_s)).astype(np.float32)
    p = nt.nt_make_partition(lengths)
    wd = weights_to_dev(w, torch)
    sd = to_dev(s, torch)
    so, zo = nt.nt_pair_block_nl(p, sd, wd, S)
    g, grads = nt.nt_pair_block_backward_nl(p, sd, zo, wd, S, _f32(gs))
    torch.cuda.synchronize()
    W64 = {k: v.f64 for k, v in w.items()}
    rs, rz = oracle.block_nl(lengths, s.f64, W64, S)
    assert scaled_max_err(f64(zo, torch), rz) <= TOL["f32"]
    assert scaled_max_err(f64(so, torch), rs) <= TOL["f32"]
    ref = oracle.block_backward_nl(lengths, s.f64, W64, S, gs.astype(np.float64))
    assert scaled_max_err(g.cpu().numpy(), ref["s"]) <= TOL["f32"]
    for k in ("Wa", "Wb", "W1", "W2", "Wo"):
        assert scaled_max_err(grads[k].cpu().numpy(), ref[k]) <= TOL["f32"], k
    assert cells > 0


def test_block_nl_full_size(nt):
    """S = 3 slices on the high-variation lengths at the four-block widths,
    the broadcast fused into the weight-stationary transition: every cell
    and single row against the oracle."""
    x = pin.workload_inputs(3, blocks=1)
    lengths = x.lengths.tolist()
    S = 3
    announce(f"non-leading block full size S={S}")
    s = pin.random_rows(sum(lengths), S * x.c_s, "bf16", seed=31)
    p = nt.nt_make_partition(lengths)
    so, zo = nt.nt_pair_block_nl(p, to_dev(s, torch), weights_to_dev(x.weights[0], torch), S)
    torch.cuda.synchronize()
    rs, rz = oracle.block_nl(lengths, s.f64, {k: v.f64 for k, v in x.weights[0].items()}, S)
    assert scaled_max_err(f64(zo, torch), rz) <= TOL["bf16"]
    assert scaled_max_err(f64(so, torch), rs) <= TOL["bf16"]
