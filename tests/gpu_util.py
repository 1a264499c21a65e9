"""Device/host conversions for the GPU tests (no block arithmetic)."""
import sys

import numpy as np

import pair_inputs as pin


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says where."""
    sys.stdout.write(f"[gpu case] {msg}\n")
    sys.stdout.flush()


def to_dev(t: pin.Tensor, torch):
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(
            torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.data)).cuda()


def weights_to_dev(w: dict, torch) -> dict:
    return {k: to_dev(v, torch) for k, v in w.items()}


def bits(x, torch) -> np.ndarray:
    """Raw storage bits of a device tensor (uint16 for bf16, uint32 for fp32)."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    if x.dtype == torch.float32:
        return x.numpy().view(np.uint32)
    return x.numpy()


def f64(x, torch) -> np.ndarray:
    """Exact float64 values of a device tensor."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return pin.bf16_bits_to_f64(x.view(torch.int16).numpy().view(np.uint16))
    return x.numpy().astype(np.float64)


def expected_bits(values64: np.ndarray, dtype: str, oracle) -> np.ndarray:
    """Storage bits of exact float64 values after one rounding to `dtype`."""
    if dtype == "bf16":
        return oracle.bf16_bits(values64)
    return np.asarray(values64, dtype=np.float64).astype(np.float32).view(np.uint32)
