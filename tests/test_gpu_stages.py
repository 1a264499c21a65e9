"""GPU parity of the three pair stages (broadcast, transition, column mean)
against the float64 oracle, on the same seeded inputs."""
import numpy as np
import pytest

import oracle
import pair_inputs as pin
from gpu_util import announce, bits, expected_bits, f64, to_dev
from helpers import TOL, scaled_max_err

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TINY = [7, 12, 5, 16]                                  # 474 cells: ragged tail of every tile
ONE_BLOCK = pin.workload_inputs(1, blocks=0).lengths.tolist()
HIGH_VAR = pin.workload_inputs(3, blocks=0).lengths.tolist()
LONG = [1024, 768, 384, 96]
EDGE = [0, 3, 0, 1, 17, 0]


@pytest.fixture(scope="module", autouse=True)
def nt():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import padding_free_pair_amd as nt
    nt._native.lib()
    return nt


def _guarded(n_rows, width, dtype, pad=64, fill=-7.0):
    """A tensor with sentinel rows around it; returns (full, view)."""
    full = torch.full((n_rows + 2 * pad, width), fill, dtype=dtype, device="cuda")
    return full, full[pad:pad + n_rows]


def _check_guard(full, pad, n_rows, fill=-7.0):
    f = full.float().cpu()
    assert (f[:pad] == fill).all() and (f[pad + n_rows:] == fill).all(), "write outside output"


TD = {"bf16": torch.bfloat16, "f32": torch.float32}


# ------------------------------------------------------------------ broadcast
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lengths,c_z", [(TINY, 8), (TINY, 24), (ONE_BLOCK, 64), (EDGE, 128),
                                         (HIGH_VAR, 128), ([300], 512), ([1] * 70, 16)])
def test_broadcast_bit_exact(nt, lengths, c_z, dtype):
    announce(f"broadcast {dtype} c_z={c_z} B={len(lengths)}")
    T = sum(lengths)
    a = pin.random_rows(T, c_z, dtype, seed=1)
    b = pin.random_rows(T, c_z, dtype, seed=2, scale=3.0)
    p = nt.nt_make_partition(lengths)
    full, z = _guarded(p.cells, c_z, TD[dtype])
    nt.nt_pair_broadcast(p, to_dev(a, torch), to_dev(b, torch), z)
    torch.cuda.synchronize()
    _check_guard(full, 64, p.cells)
    want = expected_bits(oracle.broadcast(lengths, a.f64, b.f64), dtype, oracle)
    np.testing.assert_array_equal(bits(z, torch), want)


def test_broadcast_full_size(nt):
    """The broadcast over the long-square lengths (1,795,072 cells), every
    cell bit for bit."""
    lengths, c_z = LONG, 128
    announce("broadcast full size, long square lengths")
    T = sum(lengths)
    a = pin.random_rows(T, c_z, "bf16", seed=3)
    b = pin.random_rows(T, c_z, "bf16", seed=4)
    p = nt.nt_make_partition(lengths)
    z = nt.nt_pair_broadcast(p, to_dev(a, torch), to_dev(b, torch))
    torch.cuda.synchronize()
    want = oracle.bf16_bits(oracle.broadcast(lengths, a.f64, b.f64))
    np.testing.assert_array_equal(bits(z, torch), want)


# ----------------------------------------------------------------- transition
def _mlp(c_z, hidden, dtype, seed):
    W1 = pin.random_rows(hidden, c_z, dtype, seed=seed, scale=1.0 / np.sqrt(c_z))
    W2 = pin.random_rows(c_z, hidden, dtype, seed=seed + 1, scale=1.0 / np.sqrt(hidden))
    return W1, W2


@pytest.mark.parametrize("lengths,c_z,hidden,dtype", [
    (TINY, 128, 512, "bf16"),        # MFMA path, ragged tail
    ([40, 3], 128, 512, "bf16"),
    (ONE_BLOCK, 64, 128, "bf16"),    # MFMA path, one-block widths
    (EDGE, 64, 96, "bf16"),
    (TINY, 48, 40, "bf16"),          # generic path
    (TINY, 8, 16, "f32"),            # tiny fp32 widths
    ([20, 9], 32, 64, "f32"),
    ([11], 128, 512, "f32"),
])
def test_transition_parity(nt, lengths, c_z, hidden, dtype):
    announce(f"transition {dtype} c_z={c_z} hidden={hidden} B={len(lengths)}")
    cells = int(np.sum(np.square(lengths)))
    z = pin.random_pair_rows(lengths, c_z, dtype, seed=5)
    W1, W2 = _mlp(c_z, hidden, dtype, seed=6)
    p = nt.nt_make_partition(lengths)
    zd = to_dev(z, torch)
    full, out = _guarded(cells, c_z, TD[dtype])
    nt.nt_pair_transition(p, zd, to_dev(W1, torch), to_dev(W2, torch), z_out=out)
    # in place gives the same bits
    nt.nt_pair_transition(p, zd, to_dev(W1, torch), to_dev(W2, torch), z_out=zd)
    torch.cuda.synchronize()
    _check_guard(full, 64, cells)
    np.testing.assert_array_equal(bits(out, torch), bits(zd, torch))
    ref = oracle.transition(z.f64, W1.f64, W2.f64)
    err = scaled_max_err(f64(out, torch), ref)
    assert err <= TOL[dtype], err


def test_transition_full_size(nt):
    """The unfused transition over the long-square lengths, every cell."""
    lengths, c_z, hidden = LONG, 128, 512
    announce("transition full size, long square lengths")
    z = pin.random_pair_rows(lengths, c_z, "bf16", seed=7)
    W1, W2 = _mlp(c_z, hidden, "bf16", seed=8)
    p = nt.nt_make_partition(lengths)
    out = nt.nt_pair_transition(p, to_dev(z, torch), to_dev(W1, torch), to_dev(W2, torch))
    torch.cuda.synchronize()
    ref = oracle.transition(z.f64, W1.f64, W2.f64)
    assert scaled_max_err(f64(out, torch), ref) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("c_z,hidden", [(128, 512), (64, 128), (16, 24)])
def test_transition_exact(nt, dtype, c_z, hidden):
    lengths = [2, 4, 8, 16, 1]
    announce(f"transition exact {dtype} c_z={c_z}")
    x = pin.exact_inputs(lengths, 16, c_z, hidden, dtype, seed=3)
    w = {k: v.f64 for k, v in x.weights[0].items()}
    z64 = oracle.broadcast(lengths, oracle.project(x.s.f64, w["Wa"]),
                           oracle.project(x.s.f64, w["Wb"]))
    zt = pin.store(z64, dtype)   # integers: exact in both dtypes
    p = nt.nt_make_partition(lengths)
    out = nt.nt_pair_transition(p, to_dev(zt, torch), to_dev(x.weights[0]["W1"], torch),
                                to_dev(x.weights[0]["W2"], torch))
    torch.cuda.synchronize()
    want = expected_bits(oracle.transition(z64, w["W1"], w["W2"]), dtype, oracle)
    np.testing.assert_array_equal(bits(out, torch), want)


# ----------------------------------------------------------------- column mean
@pytest.mark.parametrize("lengths,c_z,dtype", [
    (LONG, 128, "bf16"), (HIGH_VAR, 128, "bf16"), (ONE_BLOCK, 64, "bf16"), (TINY, 8, "f32"),
    (TINY, 24, "bf16"), (TINY, 24, "f32"), ([300, 5], 512, "bf16"), ([300, 5], 512, "f32"),
    (EDGE, 128, "bf16"), ([255, 256, 257, 1], 64, "f32"), ([1], 8, "bf16"),
    # widths of several power-of-two slices (three of 16, 32, 4 or 8 vectors),
    # on long rows (one workgroup a row) and short ones
    ([300, 5], 384, "bf16"), ([300, 5], 384, "f32"), (TINY, 96, "bf16"), ([257, 40], 192, "bf16"),
    (EDGE, 384, "bf16"),
])
def test_reduce_parity(nt, lengths, c_z, dtype):
    announce(f"reduce {dtype} c_z={c_z} B={len(lengths)}")
    z = pin.random_pair_rows(lengths, c_z, dtype, seed=9)
    p = nt.nt_make_partition(lengths)
    full, m = _guarded(p.T, c_z, torch.float32)
    zd = to_dev(z, torch)
    nt.nt_pair_reduce(p, zd, m=m)
    m2 = nt.nt_pair_reduce(p, zd)
    torch.cuda.synchronize()
    _check_guard(full, 64, p.T)
    np.testing.assert_array_equal(bits(m, torch), bits(m2, torch))  # deterministic
    ref = oracle.reduce_mean(lengths, z.f64)
    # inputs are exact in the storage type; only fp32 accumulation remains
    assert scaled_max_err(f64(m, torch), ref) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("c_z", [128, 24, 384])
def test_reduce_exact(nt, dtype, c_z):
    lengths = [2, 4, 8, 16, 1, 256, 512]
    announce(f"reduce exact {dtype} c_z={c_z}")
    rng = np.random.default_rng(11)
    cells = int(np.sum(np.square(lengths)))
    z = pin.store(rng.integers(-40, 41, (cells, c_z)).astype(np.float64), dtype)
    p = nt.nt_make_partition(lengths)
    m = nt.nt_pair_reduce(p, to_dev(z, torch))
    torch.cuda.synchronize()
    want = oracle.reduce_mean(lengths, z.f64).astype(np.float32).view(np.uint32)
    np.testing.assert_array_equal(bits(m, torch), want)


# ------------------------------------------------- fused broadcast + transition
@pytest.mark.parametrize("lengths,c_z,hidden,dtype", [
    (TINY, 128, 512, "bf16"), (ONE_BLOCK, 64, 128, "bf16"), (EDGE, 48, 40, "bf16"),
    (TINY, 8, 16, "f32"), ([9, 30], 32, 64, "f32"),
])
def test_broadcast_transition_parity(nt, lengths, c_z, hidden, dtype):
    announce(f"broadcast+transition {dtype} c_z={c_z} hidden={hidden} B={len(lengths)}")
    T = sum(lengths)
    a = pin.random_rows(T, c_z, "f32", seed=12)
    b = pin.random_rows(T, c_z, "f32", seed=13)
    W1, W2 = _mlp(c_z, hidden, dtype, seed=14)
    p = nt.nt_make_partition(lengths)
    full, out = _guarded(p.cells, c_z, TD[dtype])
    nt.nt_pair_broadcast_transition(p, to_dev(a, torch), to_dev(b, torch), to_dev(W1, torch),
                                    to_dev(W2, torch), z_out=out)
    torch.cuda.synchronize()
    _check_guard(full, 64, p.cells)
    ref = oracle.transition(oracle.broadcast(lengths, a.f64, b.f64), W1.f64, W2.f64)
    assert scaled_max_err(f64(out, torch), ref) <= TOL[dtype]


def test_broadcast_transition_ragged_blocks(nt):
    """The fused c_z = 128, hidden = 512 form (the weight-stationary kernel)
    on a multi-block ragged batch whose blocks mix short and long rows."""
    lengths = [3, 40, 1, 17, 64, 5, 33, 2, 29, 8]
    announce(f"broadcast+transition ragged blocks B={len(lengths)}")
    T = sum(lengths)
    a = pin.random_rows(T, 128, "f32", seed=21)
    b = pin.random_rows(T, 128, "f32", seed=22)
    W1, W2 = _mlp(128, 512, "bf16", seed=23)
    p = nt.nt_make_partition(lengths)
    full, out = _guarded(p.cells, 128, TD["bf16"])
    nt.nt_pair_broadcast_transition(p, to_dev(a, torch), to_dev(b, torch), to_dev(W1, torch),
                                    to_dev(W2, torch), z_out=out)
    torch.cuda.synchronize()
    _check_guard(full, 64, p.cells)
    ref = oracle.transition(oracle.broadcast(lengths, a.f64, b.f64), W1.f64, W2.f64)
    assert scaled_max_err(f64(out, torch), ref) <= TOL["bf16"]


@pytest.mark.parametrize("idx", [3, 4])
def test_broadcast_transition_full_size(nt, idx):
    """The fused kernel at a full workload size, where every workgroup runs
    many blocks (and stages each next block during the current one), checked
    on every cell against the oracle."""
    x = pin.workload_inputs(idx)
    lengths = x.lengths.tolist()
    announce(f"broadcast+transition full size {x.name}")
    T = sum(lengths)
    a = pin.random_rows(T, 128, "f32", seed=31)
    b = pin.random_rows(T, 128, "f32", seed=32)
    W1, W2 = _mlp(128, 512, "bf16", seed=33)
    p = nt.nt_make_partition(lengths)
    full, out = _guarded(p.cells, 128, TD["bf16"])
    nt.nt_pair_broadcast_transition(p, to_dev(a, torch), to_dev(b, torch), to_dev(W1, torch),
                                    to_dev(W2, torch), z_out=out)
    torch.cuda.synchronize()
    _check_guard(full, 64, p.cells)
    got = f64(out, torch)
    ref = oracle.transition(oracle.broadcast(lengths, a.f64, b.f64), W1.f64, W2.f64)
    assert scaled_max_err(got, ref) <= TOL["bf16"]


@pytest.mark.parametrize("lengths", [
    [90],          # 8,100 cells: 254 blocks of 32, fewer than one per CU
    [91],          # 8,281 cells: 259 blocks, two to a workgroup
    [128, 3],      # 16,393 cells: 513 blocks, a one-cell tail
    [181, 1, 0],   # 32,762 cells: 1,024 blocks minus a ragged tail
])
def test_broadcast_transition_block_ranges(nt, lengths):
    """The fused 128/512 kernel hands each workgroup a contiguous range of
    32-cell blocks and numbers the ranges by XCD: grids of fewer blocks than
    CUs, just over one per CU and several per CU, checked on every cell."""
    announce(f"broadcast+transition block ranges {lengths}")
    T = sum(lengths)
    a = pin.random_rows(T, 128, "f32", seed=51)
    b = pin.random_rows(T, 128, "f32", seed=52)
    W1, W2 = _mlp(128, 512, "bf16", seed=53)
    p = nt.nt_make_partition(lengths)
    full, out = _guarded(p.cells, 128, TD["bf16"])
    nt.nt_pair_broadcast_transition(p, to_dev(a, torch), to_dev(b, torch), to_dev(W1, torch),
                                    to_dev(W2, torch), z_out=out)
    torch.cuda.synchronize()
    _check_guard(full, 64, p.cells)
    ref = oracle.transition(oracle.broadcast(lengths, a.f64, b.f64), W1.f64, W2.f64)
    assert scaled_max_err(f64(out, torch), ref) <= TOL["bf16"]


def test_broadcast_transition_repeatable(nt):
    """The fused 128/512 kernel sums the four waves' partials in a fixed order
    (no atomics): three launches on the full high-variation workload give the
    same bits."""
    x = pin.workload_inputs(3)
    lengths = x.lengths.tolist()
    announce("broadcast+transition repeatable, high_variation_x4")
    T = sum(lengths)
    a = to_dev(pin.random_rows(T, 128, "f32", seed=71), torch)
    b = to_dev(pin.random_rows(T, 128, "f32", seed=72), torch)
    W1, W2 = _mlp(128, 512, "bf16", seed=73)
    W1d, W2d = to_dev(W1, torch), to_dev(W2, torch)
    p = nt.nt_make_partition(lengths)
    outs = [bits(nt.nt_pair_broadcast_transition(p, a, b, W1d, W2d), torch) for _ in range(3)]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_broadcast_transition_many_samples(nt):
    """More than 256 samples (the partition is decoded from global memory
    rather than an LDS copy) with empty and one-cell samples, at the fused
    128/512 shape; every cell against the oracle."""
    rng = np.random.default_rng(61)
    lengths = rng.integers(0, 13, 300).tolist() + [40, 1, 0, 33]
    announce(f"broadcast+transition B={len(lengths)}")
    T = sum(lengths)
    a = pin.random_rows(T, 128, "f32", seed=62)
    b = pin.random_rows(T, 128, "f32", seed=63)
    W1, W2 = _mlp(128, 512, "bf16", seed=64)
    p = nt.nt_make_partition(lengths)
    full, out = _guarded(p.cells, 128, TD["bf16"])
    nt.nt_pair_broadcast_transition(p, to_dev(a, torch), to_dev(b, torch), to_dev(W1, torch),
                                    to_dev(W2, torch), z_out=out)
    torch.cuda.synchronize()
    _check_guard(full, 64, p.cells)
    ref = oracle.transition(oracle.broadcast(lengths, a.f64, b.f64), W1.f64, W2.f64)
    assert scaled_max_err(f64(out, torch), ref) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("c_z,hidden", [(128, 512), (64, 128), (16, 24)])
def test_broadcast_transition_exact(nt, dtype, c_z, hidden):
    lengths = [2, 4, 8, 16, 1]
    announce(f"broadcast+transition exact {dtype} c_z={c_z}")
    x = pin.exact_inputs(lengths, 16, c_z, hidden, dtype, seed=4)
    w = {k: v.f64 for k, v in x.weights[0].items()}
    a64 = oracle.project(x.s.f64, w["Wa"])
    b64 = oracle.project(x.s.f64, w["Wb"])
    p = nt.nt_make_partition(lengths)
    out = nt.nt_pair_broadcast_transition(p, to_dev(pin.store(a64, "f32"), torch),
                                          to_dev(pin.store(b64, "f32"), torch),
                                          to_dev(x.weights[0]["W1"], torch),
                                          to_dev(x.weights[0]["W2"], torch))
    torch.cuda.synchronize()
    want = expected_bits(oracle.transition(oracle.broadcast(lengths, a64, b64), w["W1"], w["W2"]),
                         dtype, oracle)
    np.testing.assert_array_equal(bits(out, torch), want)


# ------------------------------------------- pre-normalised SwiGLU transition
def _swiglu_params(c_z, hidden, seed):
    """LN affine (fp32, gamma near 1) and gate / value / down weights (bf16)."""
    rng = np.random.default_rng(seed)
    gamma = (1.0 + 0.2 * rng.standard_normal(c_z)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(c_z)).astype(np.float32)
    Wg = pin.random_rows(hidden, c_z, "bf16", seed=seed + 1, scale=1.0 / np.sqrt(c_z))
    Wu = pin.random_rows(hidden, c_z, "bf16", seed=seed + 2, scale=1.0 / np.sqrt(c_z))
    Wd = pin.random_rows(c_z, hidden, "bf16", seed=seed + 3, scale=1.0 / np.sqrt(hidden))
    return gamma, beta, Wg, Wu, Wd


def _swiglu_dev(params):
    gamma, beta, Wg, Wu, Wd = params
    return (torch.from_numpy(gamma).cuda(), torch.from_numpy(beta).cuda(),
            to_dev(Wg, torch), to_dev(Wu, torch), to_dev(Wd, torch))


def _swiglu_ref(z64, params, eps=1e-5):
    gamma, beta, Wg, Wu, Wd = params
    return oracle.transition_swiglu(z64, gamma.astype(np.float64), beta.astype(np.float64),
                                    Wg.f64, Wu.f64, Wd.f64, eps)


@pytest.mark.parametrize("lengths,c_z,hidden", [
    (TINY, 128, 512),        # ragged tail of a single tile
    ([40, 3, 29], 128, 512),  # several tiles
    (ONE_BLOCK, 64, 128),
    (EDGE, 64, 96),           # zero-length samples, hidden not a power of two
    ([33, 18], 128, 96),
])
def test_swiglu_transition_parity(nt, lengths, c_z, hidden):
    announce(f"swiglu transition c_z={c_z} hidden={hidden} B={len(lengths)}")
    z = pin.random_pair_rows(lengths, c_z, "bf16", seed=51)
    params = _swiglu_params(c_z, hidden, seed=52)
    p = nt.nt_make_partition(lengths)
    full, out = _guarded(p.cells, c_z, torch.bfloat16)
    nt.nt_pair_transition_swiglu(p, to_dev(z, torch), *_swiglu_dev(params), z_out=out)
    torch.cuda.synchronize()
    _check_guard(full, 64, p.cells)
    err = scaled_max_err(f64(out, torch), _swiglu_ref(z.f64, params))
    announce(f"error {err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("hidden", [64, 128, 192, 256, 320, 1024])
def test_swiglu_transition_ring_phases(nt, hidden):
    """The persistent 32x32 kernel at 2, 4, 6, 8, 10 and 32 hidden chunks:
    its five-buffer weight ring meets a tile boundary at every phase (the
    chunk count mod 5: 2, 4, 1, 3, 0, 2; at two chunks the ring holds the
    same chunk twice), and 301 tiles of 256 cells give some workgroups a
    second tile, others one."""
    lengths, c_z = [256, 100, 37], 128
    announce(f"swiglu transition ring phases hidden={hidden} cells={sum(n * n for n in lengths)}")
    z = pin.random_pair_rows(lengths, c_z, "bf16", seed=61)
    params = _swiglu_params(c_z, hidden, seed=62)
    p = nt.nt_make_partition(lengths)
    full, out = _guarded(p.cells, c_z, torch.bfloat16)
    nt.nt_pair_transition_swiglu(p, to_dev(z, torch), *_swiglu_dev(params), z_out=out)
    torch.cuda.synchronize()
    _check_guard(full, 64, p.cells)
    err = scaled_max_err(f64(out, torch), _swiglu_ref(z.f64, params))
    announce(f"error {err:.3e}")
    assert err <= TOL["bf16"], err


def test_swiglu_transition_in_place_and_eps(nt):
    lengths, c_z, hidden = [21, 9, 30], 128, 512
    announce("swiglu transition in place, eps 1e-3")
    z = pin.random_pair_rows(lengths, c_z, "bf16", seed=53)
    params = _swiglu_params(c_z, hidden, seed=54)
    p = nt.nt_make_partition(lengths)
    zd = to_dev(z, torch)
    out = nt.nt_pair_transition_swiglu(p, zd, *_swiglu_dev(params), z_out=zd, ln_eps=1e-3)
    torch.cuda.synchronize()
    assert out.data_ptr() == zd.data_ptr()
    assert scaled_max_err(f64(zd, torch), _swiglu_ref(z.f64, params, 1e-3)) <= TOL["bf16"]


def test_swiglu_transition_full_size(nt):
    x = pin.workload_inputs(3)
    lengths = x.lengths.tolist()
    announce(f"swiglu transition full size {x.name}")
    z = pin.random_pair_rows(lengths, 128, "bf16", seed=55)
    params = _swiglu_params(128, 512, seed=56)
    p = nt.nt_make_partition(lengths)
    out = nt.nt_pair_transition_swiglu(p, to_dev(z, torch), *_swiglu_dev(params))
    torch.cuda.synchronize()
    assert scaled_max_err(f64(out, torch), _swiglu_ref(z.f64, params)) <= TOL["bf16"]


def test_broadcast_transition_beyond_buffer_range(nt):
    """More than 2^22 single rows: a and b (fp32, 512 bytes a row) no longer
    fit the 32-bit buffer range the weight-stationary kernel addresses them
    with, and the fused 128/512 form runs the persistent kernel instead (its
    partition decoded from global memory: 2,097,153 samples). Lengths 1, 2
    and 3 in turn; sampled cells, first and last cells of samples and the
    ragged end against the oracle."""
    k = 699051
    lengths = [1, 2, 3] * k + [1, 2, 3]
    T = sum(lengths)
    assert T > (2 ** 31 - 1) // 512
    announce(f"broadcast+transition beyond the buffer range T={T}")
    a = pin.random_rows(T, 128, "f32", seed=61)
    b = pin.random_rows(T, 128, "f32", seed=62)
    W1, W2 = _mlp(128, 512, "bf16", seed=63)
    p = nt.nt_make_partition(lengths)
    out = nt.nt_pair_broadcast_transition(p, to_dev(a, torch), to_dev(b, torch),
                                          to_dev(W1, torch), to_dev(W2, torch))
    torch.cuda.synchronize()
    o = np.concatenate([[0], np.cumsum(np.square(np.asarray(lengths, dtype=np.int64)))])
    rng = np.random.default_rng(64)
    ids = np.unique(np.concatenate([rng.integers(0, p.cells, 20000), o[:2000], o[-2000:-1],
                                    np.arange(p.cells - 300, p.cells)]))
    got = f64(out[torch.from_numpy(ids).cuda()], torch)
    ref = oracle.transition(oracle.broadcast_cells(lengths, a.f64, b.f64, ids), W1.f64, W2.f64)
    assert scaled_max_err(got, ref) <= TOL["bf16"]
