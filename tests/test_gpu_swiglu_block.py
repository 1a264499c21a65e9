"""GPU parity of the block with the paper's own transition, the residual
pre-normalised SwiGLU (DanLing NestedTensor, Equation 1 with h o LN_{C_p};
Appendix A.1, expansion four), through nt_pair_block_ex, nt_pair_chain_ex
and nt_pair_block_backward_ex, against oracle.block_swiglu,
oracle.chain_swiglu and the oracle's SwiGLU gradients (bf16: 2e-2 scaled
max error). The transition is smooth, so every gradient element is compared
at the tolerance with no decision to fit."""
import numpy as np
import pytest

import oracle
import pair_inputs as pin
from gpu_util import announce, bits, f64, to_dev, weights_to_dev
from helpers import TOL, scaled_max_err

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ORACLE_KEYS = {"W_gate": "Wg", "W_up": "Wu", "W_down": "Wd"}


@pytest.fixture(scope="module", autouse=True)
def nt():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import padding_free_pair_amd as nt
    nt._native.lib()  # raises if the library is missing: no fallback
    return nt


def _w64(w):
    return {ORACLE_KEYS.get(k, k): v.f64 for k, v in w.items()}


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("lengths,c_s,c_z,hidden", [
    ([7, 0, 33, 1, 12], 64, 128, 512),      # the pages' widths, ragged tiles, an empty sample
    ([9, 40, 2], 128, 64, 128),             # c_z 64
    ([300], 32, 128, 96),                    # one long sample, hidden not a power of two
])
def test_swiglu_block_matches_oracle(nt, lengths, c_s, c_z, hidden):
    announce(f"swiglu block {lengths} c_s={c_s} c_z={c_z} hidden={hidden}")
    x = pin.make_swiglu_inputs(lengths, c_s, c_z, hidden, "bf16", seed=3)
    p = nt.nt_make_partition(lengths)
    s_out, z_out = nt.nt_pair_block_ex(p, to_dev(x.s, torch), weights_to_dev(x.weights[0], torch))
    torch.cuda.synchronize()
    rs, rz = oracle.block_swiglu(lengths, x.s.f64, _w64(x.weights[0]))
    assert scaled_max_err(f64(z_out, torch), rz) <= TOL["bf16"]
    assert scaled_max_err(f64(s_out, torch), rs) <= TOL["bf16"]


@pytest.mark.parametrize("hidden", [64, 192, 256, 320, 1024])
def test_swiglu_block_ring_phases(nt, hidden):
    """The fused kernel at 2, 6, 8, 10 and 32 hidden chunks over 301 tiles of
    256 cells: its five-buffer weight ring meets tile boundaries at every
    phase (the chunk count mod 5), and some workgroups take a second tile."""
    lengths, c_s, c_z = [256, 100, 37], 64, 128
    announce(f"swiglu block ring phases hidden={hidden}")
    x = pin.make_swiglu_inputs(lengths, c_s, c_z, hidden, "bf16", seed=12)
    p = nt.nt_make_partition(lengths)
    s_out, z_out = nt.nt_pair_block_ex(p, to_dev(x.s, torch), weights_to_dev(x.weights[0], torch))
    torch.cuda.synchronize()
    rs, rz = oracle.block_swiglu(lengths, x.s.f64, _w64(x.weights[0]))
    assert scaled_max_err(f64(z_out, torch), rz) <= TOL["bf16"]
    assert scaled_max_err(f64(s_out, torch), rs) <= TOL["bf16"]


def test_swiglu_block_eps_and_many_samples(nt):
    """300 samples (two-launch partition, cells decoded over many samples per
    tile) and a larger LN epsilon."""
    rng = np.random.default_rng(5)
    lengths = rng.integers(0, 9, 300).tolist()
    announce(f"swiglu block B={len(lengths)} eps=1e-3")
    x = pin.make_swiglu_inputs(lengths, 32, 64, 128, "bf16", seed=4)
    p = nt.nt_make_partition(lengths)
    s_out, z_out = nt.nt_pair_block_ex(p, to_dev(x.s, torch), weights_to_dev(x.weights[0], torch),
                                       ln_eps=1e-3)
    torch.cuda.synchronize()
    rs, rz = oracle.block_swiglu(lengths, x.s.f64, _w64(x.weights[0]), eps=1e-3)
    assert scaled_max_err(f64(z_out, torch), rz) <= TOL["bf16"]
    assert scaled_max_err(f64(s_out, torch), rs) <= TOL["bf16"]


def test_relu_kind_is_the_block(nt):
    """nt_pair_block_ex with the ReLU MLP's parameters launches nt_pair_block's
    kernels: the same bits."""
    lengths = [9, 30, 2, 0, 17]
    announce("block_ex relu kind against nt_pair_block")
    x = pin.make_inputs(lengths, 384, 128, 512, "bf16", seed=7)
    p = nt.nt_make_partition(lengths)
    w = weights_to_dev(x.weights[0], torch)
    sd = to_dev(x.s, torch)
    s_a, z_a = nt.nt_pair_block(p, sd, w)
    s_b, z_b = nt.nt_pair_block_ex(p, sd, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(s_b, torch), bits(s_a, torch))
    np.testing.assert_array_equal(bits(z_b, torch), bits(z_a, torch))


def test_swiglu_block_rectangular(nt):
    rows, cols = [7, 12, 0, 5, 16], [3, 20, 4, 5, 1]
    announce("swiglu block rectangular")
    x = pin.make_swiglu_inputs(rows, 64, 128, 512, "bf16", seed=8)
    xc = pin.random_rows(sum(cols), 64, "bf16", seed=9)
    p = nt.nt_make_partition_rect(rows, cols)
    w = weights_to_dev(x.weights[0], torch)
    s_out, z_out = nt.nt_pair_block_ex(p, to_dev(x.s, torch), w, s_cols=to_dev(xc, torch))
    torch.cuda.synchronize()
    # the oracle's rectangular block with the SwiGLU transition, composed from
    # its steps: row and column projections, broadcast, transition, mean / M_i
    W = _w64(x.weights[0])
    a = oracle.project(x.s.f64, W["Wa"])
    b = oracle.project(xc.f64, W["Wb"])
    z = oracle.broadcast_rect(rows, cols, a, b)
    zt = oracle.transition_swiglu(z, W["ln_gamma"], W["ln_beta"], W["Wg"], W["Wu"], W["Wd"])
    m = oracle.reduce_mean_rect(rows, cols, zt)
    rs = x.s.f64 + oracle.project(m, W["Wo"])
    assert scaled_max_err(f64(z_out, torch), zt) <= TOL["bf16"]
    assert scaled_max_err(f64(s_out, torch), rs) <= TOL["bf16"]


def test_swiglu_chain_matches_oracle(nt):
    lengths = [13, 1, 40, 0, 27]
    announce("swiglu chain of three blocks")
    x = pin.make_swiglu_inputs(lengths, 64, 128, 512, "bf16", blocks=3, seed=10)
    p = nt.nt_make_partition(lengths)
    s_out, z_out = nt.nt_pair_chain_ex(p, to_dev(x.s, torch),
                                       [weights_to_dev(w, torch) for w in x.weights])
    torch.cuda.synchronize()
    rs, rz = oracle.chain_swiglu(lengths, x.s.f64, [_w64(w) for w in x.weights])
    assert scaled_max_err(f64(z_out, torch), rz) <= TOL["bf16"]
    assert scaled_max_err(f64(s_out, torch), rs) <= TOL["bf16"]


def test_swiglu_chain_full_size_per_block(nt):
    """Four SwiGLU blocks at the high-variation workload's lengths and
    widths, launched as a chain would launch them, each block against the
    oracle on its GPU inputs: every cell and single row."""
    w = pin.workload("high_variation_x4")
    L = pin.workload_inputs(w.index).lengths.tolist()
    x = pin.make_swiglu_inputs(L, w.c_s, w.c_z, w.hidden, "bf16", blocks=4, seed=11)
    p = nt.nt_make_partition(L)
    s = to_dev(x.s, torch)
    z_out = torch.empty((p.cells, w.c_z), dtype=torch.bfloat16, device="cuda")
    for k, wk in enumerate(x.weights):
        announce(f"swiglu chain full size block {k}")
        s_in64 = f64(s, torch)
        s_next, _ = nt.nt_pair_block_ex(p, s, weights_to_dev(wk, torch), z_out=z_out)
        torch.cuda.synchronize()
        rs, rz = oracle.block_swiglu(L, s_in64, _w64(wk))
        ez = scaled_max_err(f64(z_out, torch), rz)
        es = scaled_max_err(f64(s_next, torch), rs)
        announce(f"errors z={ez:.3e} s={es:.3e}")
        assert ez <= TOL["bf16"] and es <= TOL["bf16"]
        s = s_next


def test_swiglu_block_full_size_long_square(nt):
    """One SwiGLU block at the long-square workload's lengths and widths
    (1,795,072 cells; 7,012 tiles over the persistent grid): every cell and
    single row against the oracle."""
    w = pin.workload("long_square_x4")
    L = pin.workload_inputs(w.index).lengths.tolist()
    announce(f"swiglu block full size {w.name}")
    x = pin.make_swiglu_inputs(L, w.c_s, w.c_z, w.hidden, "bf16", blocks=1, seed=13)
    p = nt.nt_make_partition(L)
    s_out, z_out = nt.nt_pair_block_ex(p, to_dev(x.s, torch), weights_to_dev(x.weights[0], torch))
    torch.cuda.synchronize()
    rs, rz = oracle.block_swiglu(L, x.s.f64, _w64(x.weights[0]))
    ez = scaled_max_err(f64(z_out, torch), rz)
    es = scaled_max_err(f64(s_out, torch), rs)
    announce(f"errors z={ez:.3e} s={es:.3e}")
    assert ez <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("lengths,c_s,c_z,hidden,with_gz", [
    ([7, 0, 12, 1, 5], 64, 128, 512, True),
    ([9, 20, 13], 384, 128, 512, False),     # the pages' widths
    ([9, 40, 2], 128, 64, 128, True),
    ([5, 33, 17], 64, 128, 256, True),       # fused gradient, 8 chunks
    ([3, 40, 11], 64, 128, 1024, False),     # fused gradient, 32 chunks
    ([9, 20], 64, 128, 192, True),           # hidden not a multiple of 128: composed gradient
])
def test_swiglu_block_backward(nt, lengths, c_s, c_z, hidden, with_gz):
    announce(f"swiglu block backward {lengths} c_s={c_s} c_z={c_z} gz={with_gz}")
    x = pin.make_swiglu_inputs(lengths, c_s, c_z, hidden, "bf16", seed=12)
    w = x.weights[0]
    cells = int(np.square(lengths).sum())
    rng = np.random.default_rng(13)
    gs = rng.standard_normal((sum(lengths), c_s)).astype(np.float32)
    gz = rng.standard_normal((cells, c_z)).astype(np.float32) if with_gz else None
    p = nt.nt_make_partition(lengths)
    wd = weights_to_dev(w, torch)
    sd = to_dev(x.s, torch)
    _, z_out = nt.nt_pair_block_ex(p, sd, wd)
    g_s, grads = nt.nt_pair_block_backward_ex(p, sd, z_out, wd, _f32(gs),
                                              None if gz is None else _f32(gz))
    torch.cuda.synchronize()
    ref = oracle.block_swiglu_backward(lengths, x.s.f64, _w64(w), gs.astype(np.float64),
                                       None if gz is None else gz.astype(np.float64))
    assert scaled_max_err(g_s.cpu().numpy(), ref["s"]) <= TOL["bf16"]
    for k in pin.SWIGLU_NAMES:
        e = scaled_max_err(grads[k].cpu().numpy(), ref[ORACLE_KEYS.get(k, k)])
        assert e <= TOL["bf16"], (k, e)


def test_swiglu_chain_backward_under_eq5(nt):
    """Two SwiGLU blocks and Equation 5 as a training step launches them: the
    loss and its gradients against the oracle's Equation 5 on the GPU's
    outputs, then each block's gradients against the oracle on that block's
    own GPU inputs and incoming gradient (so bf16 rounding does not compound
    across the blocks)."""
    lengths = [9, 1, 24, 0, 13]
    announce("swiglu chain backward under eq5")
    x = pin.make_swiglu_inputs(lengths, 64, 128, 512, "bf16", blocks=2, seed=14)
    p = nt.nt_make_partition(lengths)
    ws = [weights_to_dev(w, torch) for w in x.weights]
    s = [to_dev(x.s, torch)]
    zs = []
    for w in ws:
        so, zo = nt.nt_pair_block_ex(p, s[-1], w)
        s.append(so)
        zs.append(zo)
    loss, g_x, g_pz = nt.nt_pair_loss_eq5(p, s[-1], zs[-1])
    g = [None, None, g_x]
    grads = [None, None]
    for k in (1, 0):
        g[k], grads[k] = nt.nt_pair_block_backward_ex(p, s[k], zs[k], ws[k], g[k + 1],
                                                      g_pz if k == 1 else None)
    torch.cuda.synchronize()
    L, rgx, rgp = oracle.loss_eq5(lengths, lengths, f64(s[-1], torch), f64(zs[-1], torch))
    assert float(loss.cpu()[0]) == pytest.approx(L, rel=1e-5)
    assert scaled_max_err(g_x.cpu().numpy(), rgx) <= 1e-6
    assert scaled_max_err(g_pz.cpu().numpy(), rgp) <= 1e-6
    for k in (1, 0):
        ref = oracle.block_swiglu_backward(lengths, f64(s[k], torch), _w64(x.weights[k]),
                                           g[k + 1].cpu().numpy().astype(np.float64),
                                           rgp if k == 1 else None)
        assert scaled_max_err(g[k].cpu().numpy(), ref["s"]) <= TOL["bf16"], k
        for name in pin.SWIGLU_NAMES:
            e = scaled_max_err(grads[k][name].cpu().numpy(), ref[ORACLE_KEYS.get(name, name)])
            assert e <= TOL["bf16"], (k, name, e)


def test_swiglu_block_backward_full_size(nt):
    """The high-variation workload's lengths and widths: every gradient."""
    w = pin.workload("high_variation_x4")
    L = pin.workload_inputs(w.index).lengths.tolist()
    announce("swiglu block backward full size")
    x = pin.make_swiglu_inputs(L, w.c_s, w.c_z, w.hidden, "bf16", seed=15)
    cells = int(np.square(np.asarray(L, dtype=np.int64)).sum())
    rng = np.random.default_rng(16)
    gs = rng.standard_normal((sum(L), w.c_s)).astype(np.float32)
    gz = (rng.standard_normal((cells, w.c_z)) / 64).astype(np.float32)
    p = nt.nt_make_partition(L)
    wd = weights_to_dev(x.weights[0], torch)
    sd = to_dev(x.s, torch)
    _, z_out = nt.nt_pair_block_ex(p, sd, wd)
    g_s, grads = nt.nt_pair_block_backward_ex(p, sd, z_out, wd, _f32(gs), _f32(gz))
    torch.cuda.synchronize()
    ref = oracle.block_swiglu_backward(L, x.s.f64, _w64(x.weights[0]), gs.astype(np.float64),
                                       gz.astype(np.float64))
    assert scaled_max_err(g_s.cpu().numpy(), ref["s"]) <= TOL["bf16"]
    for k in pin.SWIGLU_NAMES:
        e = scaled_max_err(grads[k].cpu().numpy(), ref[ORACLE_KEYS.get(k, k)])
        assert e <= TOL["bf16"], (k, e)


def test_swiglu_block_backward_deterministic(nt):
    """Two calls on the same inputs give the same bits: the LN parameters'
    sums over the cells run in a fixed order (per-workgroup sums over a
    fixed grid, then the workgroups in order), as do the weight
    contractions' slices."""
    L = [40, 3, 130, 0, 77]
    announce(f"swiglu block backward deterministic {L}")
    x = pin.make_swiglu_inputs(L, 64, 128, 512, "bf16", seed=21)
    rng = np.random.default_rng(22)
    gs = _f32(rng.standard_normal((sum(L), 64)))
    gz = _f32(rng.standard_normal((int(np.square(L).sum()), 128)))
    p = nt.nt_make_partition(L)
    wd = weights_to_dev(x.weights[0], torch)
    sd = to_dev(x.s, torch)
    _, z_out = nt.nt_pair_block_ex(p, sd, wd)
    g1, r1 = nt.nt_pair_block_backward_ex(p, sd, z_out, wd, gs, gz)
    g2, r2 = nt.nt_pair_block_backward_ex(p, sd, z_out, wd, gs, gz)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g1.cpu().numpy(), g2.cpu().numpy())
    for k in r1:
        np.testing.assert_array_equal(r1[k].cpu().numpy(), r2[k].cpu().numpy(), err_msg=k)


def test_swiglu_block_backward_empty_batch(nt):
    """No singles and no cells: every gradient is zero."""
    announce("swiglu block backward empty")
    x = pin.make_swiglu_inputs([1], 64, 128, 512, "bf16", seed=17)  # parameters only
    p = nt.nt_make_partition([0, 0])
    wd = weights_to_dev(x.weights[0], torch)
    s = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    gs = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    g, grads = nt.nt_pair_block_backward_ex(p, s, z, wd, gs)
    torch.cuda.synchronize()
    assert g.numel() == 0
    for k, v in grads.items():
        assert torch.count_nonzero(v).item() == 0, k
