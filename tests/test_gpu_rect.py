"""GPU parity for rectangular pairs (N_i x M_i): partition, decode, broadcast,
column mean and the rectangular block, against the oracle."""
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
    nt._native.lib()  # raises if the library is missing: no fallback
    return nt


def _cases():
    rng = np.random.default_rng(77)
    big_r = rng.integers(0, 30, 400)
    big_c = rng.integers(0, 30, 400)
    return [
        ([2, 0, 3], [4, 5, 1]),
        ([7, 12, 5, 16], [3, 20, 5, 1]),
        ([0, 9], [3, 0]),                 # rows without cells, cells without rows
        ([1] * 300, [2] * 300),           # more samples than the one-launch path takes
        ([300, 2], [1, 400]),             # long rows and a long column axis
        (big_r.tolist(), big_c.tolist()),
        ([16, 16], [16, 16]),             # square, through the rectangular constructor
    ]


@pytest.mark.parametrize("rows,cols", _cases(), ids=lambda v: f"B{len(v)}_{sum(v)}")
def test_rect_partition_and_decode_bit_exact(nt, rows, cols):
    announce(f"rect partition B={len(rows)} T={sum(rows)} T_cols={sum(cols)}")
    p = nt.nt_make_partition_rect(rows, cols)
    torch.cuda.synchronize()
    ref = oracle.partition_rect(rows, cols)
    assert (p.T, p.T_cols, p.cells, p.B) == (ref["T"], ref["T_cols"], ref["cells"], ref["B"])
    arr = {k: v.cpu().numpy() for k, v in p.arrays().items()}
    np.testing.assert_array_equal(arr["single_offsets"], ref["single_offsets"])
    np.testing.assert_array_equal(arr["col_offsets"], ref["col_offsets"])
    np.testing.assert_array_equal(arr["pair_offsets"], ref["pair_offsets"])
    np.testing.assert_array_equal(arr["row_splits"], ref["row_splits"])
    np.testing.assert_array_equal(arr["row_sample"], ref["row_sample"])
    np.testing.assert_array_equal(arr["lengths"], np.asarray(rows, dtype=np.int32))
    np.testing.assert_array_equal(arr["col_lengths"], np.asarray(cols, dtype=np.int32))
    o = ref["pair_offsets"]
    want_tiles = [int(np.searchsorted(o, t, side="right") - 1) for t in range(0, p.cells, 256)]
    np.testing.assert_array_equal(arr["tile_sample"], np.array(want_tiles, dtype=np.int32))
    if p.cells:
        sample, row, col = (t.cpu().numpy() for t in nt.nt_decode_cells(p))
        r_s, r_r, r_c = oracle.decode_cells_rect(rows, cols)
        np.testing.assert_array_equal(sample, r_s)
        np.testing.assert_array_equal(row, r_r)
        np.testing.assert_array_equal(col, r_c)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,c_z", [([7, 12, 5, 16], [3, 20, 5, 1], 128),
                                           ([0, 9, 4], [3, 0, 70], 24),
                                           ([300, 2], [1, 400], 64)])
def test_rect_broadcast_bit_exact(nt, rows, cols, c_z, dtype):
    announce(f"rect broadcast {dtype} c_z={c_z}")
    a = pin.random_rows(sum(rows), c_z, dtype, seed=1)
    b = pin.random_rows(sum(cols), c_z, dtype, seed=2, scale=3.0)
    p = nt.nt_make_partition_rect(rows, cols)
    z = nt.nt_pair_broadcast(p, to_dev(a, torch), to_dev(b, torch))
    torch.cuda.synchronize()
    want = expected_bits(oracle.broadcast_rect(rows, cols, a.f64, b.f64), dtype, oracle)
    np.testing.assert_array_equal(bits(z, torch), want)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("c_z", [128, 24])
def test_rect_reduce_exact(nt, dtype, c_z):
    # power-of-two column counts divide exactly; a sample with M_i = 0 has
    # rows without cells, whose mean is 0/0 on both sides
    rows, cols = [3, 5, 2, 7, 4], [2, 256, 0, 512, 16]
    announce(f"rect reduce exact {dtype} c_z={c_z}")
    rng = np.random.default_rng(12)
    cells = int(np.dot(rows, cols))
    z = pin.store(rng.integers(-40, 41, (cells, c_z)).astype(np.float64), dtype)
    p = nt.nt_make_partition_rect(rows, cols)
    m = nt.nt_pair_reduce(p, to_dev(z, torch))
    torch.cuda.synchronize()
    ref = oracle.reduce_mean_rect(rows, cols, z.f64)
    got = m.cpu().numpy()
    assert np.isnan(got).sum() == np.isnan(ref).sum() == 2 * c_z
    keep = ~np.isnan(ref)
    np.testing.assert_array_equal(got[keep].view(np.uint32),
                                  ref[keep].astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("rows,cols,c_s,c_z,hidden,dtype", [
    ([7, 12, 5, 16], [3, 20, 5, 1], 32, 128, 512, "bf16"),  # weight-stationary fused kernel
    ([9, 40, 2], [33, 6, 64], 32, 64, 128, "bf16"),          # persistent fused kernel
    ([7, 12, 5], [3, 20, 6], 16, 48, 40, "bf16"),            # generic kernel
    ([7, 12, 5], [3, 20, 6], 16, 8, 16, "f32"),
])
def test_rect_block_matches_oracle(nt, rows, cols, c_s, c_z, hidden, dtype):
    announce(f"rect block {dtype} c_z={c_z} hidden={hidden}")
    x_r = pin.random_rows(sum(rows), c_s, dtype, seed=31)
    x_c = pin.random_rows(sum(cols), c_s, dtype, seed=32)
    scale = {"Wa": c_s, "Wb": c_s, "W1": c_z, "W2": hidden, "Wo": c_z}
    shapes = {"Wa": (c_z, c_s), "Wb": (c_z, c_s), "W1": (hidden, c_z), "W2": (c_z, hidden),
              "Wo": (c_s, c_z)}
    w = {k: pin.random_rows(*shapes[k], dtype, seed=40 + i, scale=1.0 / np.sqrt(scale[k]))
         for i, k in enumerate(shapes)}
    p = nt.nt_make_partition_rect(rows, cols)
    s_out, z_out = nt.nt_pair_block_rect(p, to_dev(x_r, torch), to_dev(x_c, torch),
                                         weights_to_dev(w, torch))
    torch.cuda.synchronize()
    ref_s, ref_z = oracle.block_rect(rows, cols, x_r.f64, x_c.f64, {k: v.f64 for k, v in w.items()})
    assert scaled_max_err(f64(z_out, torch), ref_z) <= TOL[dtype]
    assert scaled_max_err(f64(s_out, torch), ref_s) <= TOL[dtype]


def test_rect_block_with_equal_axes_is_the_square_block(nt):
    lengths = [7, 12, 5, 16, 33]
    announce("rect block with N = M against the square block")
    x = pin.workload_inputs(1, blocks=1)
    T = sum(lengths)
    s = pin.random_rows(T, x.c_s, x.dtype, seed=5)
    w = weights_to_dev(x.weights[0], torch)
    sd = to_dev(s, torch)
    s_sq, z_sq = nt.nt_pair_block(nt.nt_make_partition(lengths), sd, w)
    s_re, z_re = nt.nt_pair_block_rect(nt.nt_make_partition_rect(lengths, lengths), sd, sd, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(z_re, torch), bits(z_sq, torch))
    np.testing.assert_array_equal(bits(s_re, torch), bits(s_sq, torch))


def test_rect_block_full_size(nt):
    """Rows from the high-variation lengths, columns from the same lengths in
    reverse order (so N_i != M_i almost everywhere), at the four-block
    widths; every cell and row against the oracle."""
    x = pin.workload_inputs(3)
    rows = x.lengths.tolist()
    cols = rows[::-1]
    announce(f"rect block full size {x.name}")
    x_c = pin.random_rows(sum(cols), x.c_s, x.dtype, seed=8)
    p = nt.nt_make_partition_rect(rows, cols)
    w = weights_to_dev(x.weights[0], torch)
    s_out, z_out = nt.nt_pair_block_rect(p, to_dev(x.s, torch), to_dev(x_c, torch), w)
    torch.cuda.synchronize()
    w64 = {k: v.f64 for k, v in x.weights[0].items()}
    ref_s, ref_z = oracle.block_rect(rows, cols, x.s.f64, x_c.f64, w64)
    assert scaled_max_err(f64(z_out, torch), ref_z) <= TOL["bf16"]
    assert scaled_max_err(f64(s_out, torch), ref_s) <= TOL["bf16"]
