"""GPU parity of the whole block (nt_pair_block) and of the four-block chain
against the float64 oracle."""
import numpy as np
import pytest

import oracle
import pair_inputs as pin
from gpu_util import announce, bits, expected_bits, f64, to_dev, weights_to_dev
from helpers import TOL, scaled_max_err

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def nt():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import padding_free_pair_amd as nt
    nt._native.lib()
    return nt


def _w64(w):
    return {k: v.f64 for k, v in w.items()}


@pytest.mark.parametrize("idx", [0, 1])
def test_block_small_workloads_full(nt, idx):
    x = pin.workload_inputs(idx)
    L = x.lengths.tolist()
    announce(f"block workload {x.name}")
    p = nt.nt_make_partition(L)
    s_out, z_out = nt.nt_pair_block(p, to_dev(x.s, torch), weights_to_dev(x.weights[0], torch))
    torch.cuda.synchronize()
    ref_s, ref_z = oracle.block(L, x.s.f64, _w64(x.weights[0]))
    tol = TOL[x.dtype]
    ez = scaled_max_err(f64(z_out, torch), ref_z)
    es = scaled_max_err(f64(s_out, torch), ref_s)
    announce(f"errors z={ez:.3e} s={es:.3e} (tol {tol})")
    assert ez <= tol and es <= tol


@pytest.mark.parametrize("lengths,c_s,c_z,hidden,dtype", [
    ([3, 0, 9, 1], 32, 128, 512, "bf16"),
    ([0], 16, 64, 128, "bf16"),
    ([5, 70], 48, 24, 40, "bf16"),
    ([6, 2], 24, 16, 8, "f32"),
    ([300], 64, 64, 128, "bf16"),
])
def test_block_edge_shapes(nt, lengths, c_s, c_z, hidden, dtype):
    announce(f"block edge {dtype} {lengths} c_s={c_s} c_z={c_z} h={hidden}")
    x = pin.make_inputs(lengths, c_s, c_z, hidden, dtype, seed=21)
    p = nt.nt_make_partition(lengths)
    s_out, z_out = nt.nt_pair_block(p, to_dev(x.s, torch), weights_to_dev(x.weights[0], torch))
    torch.cuda.synchronize()
    ref_s, ref_z = oracle.block(lengths, x.s.f64, _w64(x.weights[0]))
    assert scaled_max_err(f64(z_out, torch), ref_z) <= TOL[dtype]
    assert scaled_max_err(f64(s_out, torch), ref_s) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("c_z,hidden", [(128, 512), (64, 128), (16, 32)])
def test_block_exact(nt, dtype, c_z, hidden):
    lengths = [2, 4, 8, 16, 1]
    announce(f"block exact {dtype} c_z={c_z}")
    x = pin.exact_inputs(lengths, 32, c_z, hidden, dtype, seed=5)
    p = nt.nt_make_partition(lengths)
    sd = to_dev(x.s, torch)
    s_out, z_out = nt.nt_pair_block(p, sd, weights_to_dev(x.weights[0], torch))
    # in place on the singles gives the same bits
    s_copy = sd.clone()
    nt.nt_pair_block(p, s_copy, weights_to_dev(x.weights[0], torch), s_out=s_copy)
    torch.cuda.synchronize()
    ref_s, ref_z = oracle.block(lengths, x.s.f64, _w64(x.weights[0]))
    np.testing.assert_array_equal(bits(z_out, torch), expected_bits(ref_z, dtype, oracle))
    np.testing.assert_array_equal(bits(s_out, torch), expected_bits(ref_s, dtype, oracle))
    np.testing.assert_array_equal(bits(s_copy, torch), bits(s_out, torch))


def test_block_fused_matches_stages(nt):
    # exact inputs: the fused broadcast prologue equals broadcast + transition
    lengths = [4, 8, 16]
    announce("block fused vs staged")
    x = pin.exact_inputs(lengths, 32, 128, 512, "bf16", seed=8)
    w = _w64(x.weights[0])
    a = pin.store(oracle.project(x.s.f64, w["Wa"]), "bf16")
    b = pin.store(oracle.project(x.s.f64, w["Wb"]), "bf16")
    p = nt.nt_make_partition(lengths)
    wd = weights_to_dev(x.weights[0], torch)
    _, z_block = nt.nt_pair_block(p, to_dev(x.s, torch), wd)
    z = nt.nt_pair_broadcast(p, to_dev(a, torch), to_dev(b, torch))
    z_stage = nt.nt_pair_transition(p, z, wd["W1"], wd["W2"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(z_block, torch), bits(z_stage, torch))


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_chain_full_size_per_block(nt, idx):
    """Each block of the four-block chain at full size, launched as the
    benchmark launches it, against the oracle on that block's GPU inputs:
    every cell of the pair state and every single row."""
    x = pin.workload_inputs(idx)
    L = x.lengths.tolist()
    p = nt.nt_make_partition(L)
    s = to_dev(x.s, torch)
    z_out = torch.empty((p.cells, x.c_z), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(nt.nt_block_workspace_bytes(p, x.c_s, x.c_z, x.hidden, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    for k, wk in enumerate(x.weights):
        announce(f"chain {x.name} block {k}")
        s_in64 = f64(s, torch)
        s_next = torch.empty_like(s)
        nt.nt_pair_block(p, s, weights_to_dev(wk, torch), s_out=s_next, z_out=z_out,
                         workspace=ws)
        torch.cuda.synchronize()
        ref_s, ref_z = oracle.block(L, s_in64, _w64(wk))
        ez = scaled_max_err(f64(z_out, torch), ref_z)
        es = scaled_max_err(f64(s_next, torch), ref_s)
        announce(f"errors z={ez:.3e} s={es:.3e}")
        assert ez <= TOL["bf16"], (k, ez)
        assert es <= TOL["bf16"], (k, es)
        s = s_next


@pytest.mark.parametrize("idx", [1, 3])
def test_per_sample_launches_match_segmented(nt, idx):
    """Matched-granularity control (Appendix C.8): the same kernels issued once
    per sample, on one-sample partitions and slices of the packed buffers,
    give bit-identical singles and pair state to the segmented launch: every
    kernel's arithmetic for a cell or a row is independent of its neighbours."""
    x = pin.workload_inputs(idx)
    L = [int(n) for n in x.lengths]
    announce(f"per-sample vs segmented {x.name}")
    tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    ws_seg = [weights_to_dev(wk, torch) for wk in x.weights]
    p = nt.nt_make_partition(L)
    s_seg = to_dev(x.s, torch)
    z_seg = torch.empty((p.cells, x.c_z), dtype=tdt, device="cuda")
    for w in ws_seg:
        s_next = torch.empty_like(s_seg)
        nt.nt_pair_block(p, s_seg, w, s_out=s_next, z_out=z_seg)
        s_seg = s_next
    eta = np.concatenate([[0], np.cumsum(L)])
    o = np.concatenate([[0], np.cumsum(np.square(np.asarray(L, dtype=np.int64)))])
    s_ps = to_dev(x.s, torch)
    z_ps = torch.empty_like(z_seg)
    parts = [nt.nt_make_partition([n]) for n in L]
    for w in ws_seg:
        s_next = torch.empty_like(s_ps)
        for i, pi in enumerate(parts):
            if L[i] == 0:
                continue
            e0, e1, o0, o1 = int(eta[i]), int(eta[i + 1]), int(o[i]), int(o[i + 1])
            nt.nt_pair_block(pi, s_ps[e0:e1], w, s_out=s_next[e0:e1], z_out=z_ps[o0:o1])
        s_ps = s_next
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(s_ps, torch), bits(s_seg, torch))
    np.testing.assert_array_equal(bits(z_ps, torch), bits(z_seg, torch))


# ---------------------------------------------------------------- nt_pair_chain
@pytest.mark.parametrize("lengths,c_s,c_z,hidden,dtype,blocks", [
    ([3, 0, 17, 40, 1, 33], 384, 128, 512, "bf16", 3),  # weight-stationary transition
    ([5, 20, 0, 9], 64, 64, 128, "bf16", 2),              # persistent transition
    ([6, 2, 11], 48, 24, 40, "bf16", 2),                  # generic transition
    ([7, 12, 5], 16, 8, 16, "f32", 3),                    # fp32
    ([4], 384, 128, 512, "bf16", 1),                      # one block
])
def test_chain_matches_oracle(nt, lengths, c_s, c_z, hidden, dtype, blocks):
    announce(f"chain {dtype} {lengths} c_s={c_s} c_z={c_z} h={hidden} "
             f"blocks={blocks}")
    x = pin.make_inputs(lengths, c_s, c_z, hidden, dtype, blocks=blocks, seed=23)
    p = nt.nt_make_partition(lengths)
    s_out, z_out = nt.nt_pair_chain(p, to_dev(x.s, torch),
                                    [weights_to_dev(wk, torch) for wk in x.weights])
    torch.cuda.synchronize()
    ref_s, ref_z = oracle.chain(lengths, x.s.f64, [_w64(wk) for wk in x.weights])
    ez = scaled_max_err(f64(z_out, torch), ref_z)
    es = scaled_max_err(f64(s_out, torch), ref_s)
    announce(f"errors z={ez:.3e} s={es:.3e}")
    assert ez <= TOL[dtype] and es <= TOL[dtype]


def _block_loop(nt, p, s, ws, z):
    for w in ws:
        s_next = torch.empty_like(s)
        nt.nt_pair_block(p, s, w, s_out=s_next, z_out=z)
        s = s_next
    return s


@pytest.mark.parametrize("idx", [3, 4])
def test_chain_full_size_matches_block_loop(nt, idx):
    """The chain at full size against the same blocks called one by one (each
    of which the per-block test holds to the oracle): bit for bit."""
    x = pin.workload_inputs(idx)
    L = x.lengths.tolist()
    announce(f"chain vs block loop {x.name}")
    p = nt.nt_make_partition(L)
    ws = [weights_to_dev(wk, torch) for wk in x.weights]
    s0 = to_dev(x.s, torch)
    z_loop = torch.empty((p.cells, x.c_z), dtype=torch.bfloat16, device="cuda")
    s_loop = _block_loop(nt, p, s0, ws, z_loop)
    s_ch, z_ch = nt.nt_pair_chain(p, s0, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(s_ch, torch), bits(s_loop, torch))
    np.testing.assert_array_equal(bits(z_ch, torch), bits(z_loop, torch))


def test_chain_one_block_is_the_block(nt):
    x = pin.make_inputs([9, 30, 2], 384, 128, 512, "bf16", seed=5)
    p = nt.nt_make_partition([9, 30, 2])
    s0, w = to_dev(x.s, torch), weights_to_dev(x.weights[0], torch)
    s_b, z_b = nt.nt_pair_block(p, s0, w)
    s_c, z_c = nt.nt_pair_chain(p, s0, [w])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(s_c, torch), bits(s_b, torch))
    np.testing.assert_array_equal(bits(z_c, torch), bits(z_b, torch))


def test_chain_in_place(nt):
    """s_out may be s_in: every row is read before it is written."""
    L = [13, 1, 64, 0, 27]
    x = pin.make_inputs(L, 384, 128, 512, "bf16", blocks=4, seed=8)
    p = nt.nt_make_partition(L)
    ws = [weights_to_dev(wk, torch) for wk in x.weights]
    s0 = to_dev(x.s, torch)
    s_ref, z_ref = nt.nt_pair_chain(p, s0, ws)
    s_io = s0.clone()
    _, z_io = nt.nt_pair_chain(p, s_io, ws, s_out=s_io)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(s_io, torch), bits(s_ref, torch))
    np.testing.assert_array_equal(bits(z_io, torch), bits(z_ref, torch))


@pytest.mark.parametrize("idx", [3])
def test_chain_per_sample_matches_segmented(nt, idx):
    """The chain run on each sample alone gives the bits of the batched chain:
    every kernel computes a row or a cell from that row or cell only."""
    x = pin.workload_inputs(idx)
    L = [int(n) for n in x.lengths]
    announce(f"chain per-sample vs segmented {x.name}")
    ws = [weights_to_dev(wk, torch) for wk in x.weights]
    p = nt.nt_make_partition(L)
    s0 = to_dev(x.s, torch)
    s_seg, z_seg = nt.nt_pair_chain(p, s0, ws)
    eta = np.concatenate([[0], np.cumsum(L)])
    o = np.concatenate([[0], np.cumsum(np.square(np.asarray(L, dtype=np.int64)))])
    s_ps = torch.empty_like(s_seg)
    z_ps = torch.empty_like(z_seg)
    for i, n in enumerate(L):
        if n == 0:
            continue
        e0, e1, o0, o1 = int(eta[i]), int(eta[i + 1]), int(o[i]), int(o[i + 1])
        nt.nt_pair_chain(nt.nt_make_partition([n]), s0[e0:e1], ws, s_out=s_ps[e0:e1],
                         z_out=z_ps[o0:o1])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(s_ps, torch), bits(s_seg, torch))
    np.testing.assert_array_equal(bits(z_ps, torch), bits(z_seg, torch))
