"""GPU parity of the padded comparator the benchmark reports its speed-up and
memory ratios against (DanLing NestedTensor, Section 4.1 "Measurement":
padding is the baseline; Table 2's caption: padding runs native PyTorch
kernels over the B x N_max^2 envelope). Its valid rows and cells, read in
packed order, must equal the oracle's chain within the bf16 bound, like the
packed path's; the padded rows and columns are masked out of the mean."""
import numpy as np
import pytest

import oracle
import pair_inputs as pin
from gpu_util import announce, f64
from helpers import TOL, scaled_max_err

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def bench():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bench
    return bench


@pytest.mark.parametrize("case", ["ragged", "high_variation_x4"])
def test_padded_comparator_matches_oracle(bench, case):
    if case == "ragged":
        # an empty sample, a one-row sample and N_max far above the others
        x = pin.make_inputs([7, 0, 33, 1, 12], 64, 128, 512, "bf16", blocks=2, seed=3)
    else:
        x = pin.workload_inputs(pin.workload(case).index)
    announce(f"padded comparator {case} B={len(x.lengths)} blocks={len(x.weights)}")
    env = bench.PaddedEnvelope(x, torch)
    S, P = env.step()
    s, z = env.valid(S, P)
    torch.cuda.synchronize()
    announce(f"padded product written in fp32 by the GEMM: {env.fp32_out}")
    L = x.lengths.tolist()
    rs, rz = oracle.chain(L, x.s.f64, [{k: v.f64 for k, v in w.items()} for w in x.weights])
    ez, es = scaled_max_err(f64(z, torch), rz), scaled_max_err(f64(s, torch), rs)
    announce(f"padded errors z={ez:.3e} s={es:.3e}")
    assert ez <= TOL["bf16"] and es <= TOL["bf16"]
    # masked columns were zeroed; padded rows of S never reach a valid cell
    N = env.N
    P4 = P.view(len(L), N, N, -1)
    for i, n in enumerate(L):
        assert torch.count_nonzero(P4[i, :, n:]).item() == 0
