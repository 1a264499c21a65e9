"""The seeded generator reproduces the workload lengths it is specified by."""
import numpy as np
import pytest

import pair_inputs as pin


@pytest.mark.parametrize("idx,lengths", [
    (0, [7, 12, 5, 16]),
    (1, [94, 97, 113, 125, 66, 73, 117, 125]),
    (3, [22, 36, 257, 120, 22, 72, 84, 28, 204, 24, 62, 96, 71, 122, 206, 440]),
    (4, [1024, 768, 384, 96]),
])
def test_lengths(idx, lengths):
    assert pin.workload_inputs(idx, blocks=0).lengths.tolist() == lengths


@pytest.mark.parametrize("idx,T,cells", [(0, 40, 474), (1, 810, 85638), (2, 3885, 944381),
                                         (3, 1866, 406950), (4, 2272, 1795072)])
def test_totals(idx, T, cells):
    L = pin.workload_inputs(idx, blocks=0).lengths.astype(np.int64)
    assert L.sum() == T and (L * L).sum() == cells


def test_bf16_store_is_exact_and_rne():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.1])
    t = pin.store(x, "bf16")
    assert t.f64.tolist()[:3] == [1.0, 1.0 + 2.0 ** -6, -2.5]
    assert t.data.dtype == np.uint16


def test_weights_layout_and_scale():
    x = pin.make_inputs([64] * 4, 384, 128, 512, "f32", seed=0)
    w = x.weights[0]
    assert w["Wa"].data.shape == (128, 384) and w["W1"].data.shape == (512, 128)
    assert w["W2"].data.shape == (128, 512) and w["Wo"].data.shape == (384, 128)
    # N(0, 1/fan_in): fan_in is the stored "in" (second) dimension
    for k, v in w.items():
        assert abs(v.f64.std() * np.sqrt(v.f64.shape[1]) - 1.0) < 0.05, k
