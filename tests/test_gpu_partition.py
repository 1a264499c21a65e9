"""GPU parity: partition arrays and the cell decode, bit-exact against the oracle."""
import numpy as np
import pytest

import oracle
import pair_inputs as pin
from gpu_util import announce

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
    rng = np.random.default_rng(2024)
    ragged = rng.integers(0, 40, 1000)
    ragged[rng.choice(1000, 200, replace=False)] = 0
    cases = [[2, 3], [3, 2], [1], [0], [], [0, 0, 5, 0], [1] * 300, [16] * 4,
             [255, 256, 257, 0, 1], ragged.tolist(),
             # the one-launch path takes at most 256 samples
             [3] * 255, [3] * 256, [3] * 257, [0] * 256, list(range(256))]
    cases += [pin.workload_inputs(i, blocks=0).lengths.tolist() for i in range(5)]
    return cases


@pytest.mark.parametrize("lengths", _cases(), ids=lambda L: f"B{len(L)}_T{sum(L)}")
def test_partition_bit_exact(nt, lengths):
    announce(f"partition B={len(lengths)} T={sum(lengths)}")
    p = nt.nt_make_partition(lengths)
    torch.cuda.synchronize()
    ref = oracle.partition(lengths)
    assert (p.T, p.cells, p.n_max, p.B) == (ref["T"], ref["cells"], ref["n_max"], ref["B"])
    arr = {k: v.cpu().numpy() for k, v in p.arrays().items()}
    assert arr["lengths"].tolist() == list(lengths)
    for k in ("single_offsets", "pair_offsets", "row_splits", "row_sample"):
        np.testing.assert_array_equal(arr[k], ref[k], err_msg=k)
    # tile index: the sample holding every 256th cell (Eq. 3's o_i <= t < o_{i+1})
    o = ref["pair_offsets"]
    want = [int(np.searchsorted(o, t, side="right") - 1) for t in range(0, p.cells, 256)]
    np.testing.assert_array_equal(arr["tile_sample"], np.array(want, dtype=np.int32))
    # the column-mean schedule covers every row exactly once
    items = arr["item_offsets"]
    assert items[0] == 0 and items[-1] == p.n_items
    assert (np.diff(items) >= 0).all()
    assert all((np.diff(items)[i] > 0) == (n > 0) for i, n in enumerate(lengths))


@pytest.mark.parametrize("lengths", [L for L in _cases() if sum(L)], ids=lambda L: f"B{len(L)}")
def test_decode_bit_exact(nt, lengths):
    announce(f"decode B={len(lengths)} T={sum(lengths)}")
    p = nt.nt_make_partition(lengths)
    smp, row, col = nt.nt_decode_cells(p)
    torch.cuda.synchronize()
    rs, rr, rc = oracle.decode_cells(lengths)
    np.testing.assert_array_equal(smp.cpu().numpy(), rs)
    np.testing.assert_array_equal(row.cpu().numpy(), rr)
    np.testing.assert_array_equal(col.cpu().numpy(), rc)
