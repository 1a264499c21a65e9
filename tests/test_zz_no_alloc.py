"""GPU parity of nt_pair_block_noalloc (the block with its workspace in the
library's static device scratch) against nt_pair_block, which takes a caller
workspace: the same kernels on the same inputs give the same bits. Two calls
in a row, the second on a smaller batch (the scratch keeps the first call's
contents), then the largest batch the scratch holds and one row beyond it."""
import numpy as np
import pytest

import oracle
import pair_inputs as pin
from gpu_util import announce, bits, f64, to_dev, weights_to_dev
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


def _run_both(nt, x):
    L = x.lengths.tolist()
    p = nt.nt_make_partition(L)
    wd = weights_to_dev(x.weights[0], torch)
    sd = to_dev(x.s, torch)
    s_ref, z_ref = nt.nt_pair_block(p, sd, wd)
    s_na = torch.full_like(s_ref, 7.0)
    z_na = torch.full_like(z_ref, 7.0)
    nt.nt_pair_block_noalloc(p, sd, wd, s_out=s_na, z_out=z_na)
    torch.cuda.synchronize()
    return p, s_ref, z_ref, s_na, z_na


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_block_twice(nt, dtype):
    widths = (384, 128, 512) if dtype == "bf16" else (16, 8, 16)
    for lengths in ([120, 33, 7, 0, 61, 250], [9, 20, 13]):  # the second call smaller
        announce(f"no-alloc block {dtype} {lengths}")
        x = pin.make_inputs(lengths, *widths, dtype, seed=sum(lengths))
        p, s_ref, z_ref, s_na, z_na = _run_both(nt, x)
        np.testing.assert_array_equal(bits(s_na, torch), bits(s_ref, torch))
        np.testing.assert_array_equal(bits(z_na, torch), bits(z_ref, torch))
        rs, rz = oracle.block(lengths, x.s.f64, {k: v.f64 for k, v in x.weights[0].items()})
        assert scaled_max_err(f64(z_na, torch), rz) <= TOL[dtype]
        assert scaled_max_err(f64(s_na, torch), rs) <= TOL[dtype]


def test_noalloc_limit(nt):
    # T = 10,922 rows at c_z = 128 fill the scratch (3 x 5,592,064 bytes)
    lengths = [2] * 5461
    announce(f"no-alloc block at the scratch limit T={sum(lengths)}")
    x = pin.make_inputs(lengths, 64, 128, 512, "bf16", seed=5)
    _, s_ref, z_ref, s_na, z_na = _run_both(nt, x)
    np.testing.assert_array_equal(bits(s_na, torch), bits(s_ref, torch))
    np.testing.assert_array_equal(bits(z_na, torch), bits(z_ref, torch))
    # one single row more is rejected before anything is enqueued
    lengths = lengths + [1]
    x = pin.make_inputs(lengths, 64, 128, 512, "bf16", seed=6)
    p = nt.nt_make_partition(lengths)
    wd = weights_to_dev(x.weights[0], torch)
    s_out = torch.full((p.T, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nt.NtError) as e:
        nt.nt_pair_block_noalloc(p, to_dev(x.s, torch), wd, s_out=s_out)
    assert e.value.status == nt._native.NT_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((s_out == 3.0).all())
