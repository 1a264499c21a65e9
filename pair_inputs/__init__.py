"""Seeded synthetic inputs for the packed single-pair-single block.

This module is shared by the CPU oracle and the GPU path. It draws random
numbers and stores them in the dtype a workload asks for; it performs none of
the block's arithmetic (no projection, broadcast, transition or reduction).

Workloads follow the length regimes of the DanLing NestedTensor paper
(arXiv 2609.30379): its single-pair-single block (Section 3, Equation 1) and
its four-block Pairformer-style application (Section 4.3), whose square
regimes run from near-uniform to high-variation lengths. The paper's own
length manifests are not printed, so the regimes below are drawn from seeded
distributions instead.

Layout conventions (shared by both sides, fixed here once):
  * singles ``s``: [T, c_s] row-major, samples concatenated in batch order;
  * weights are stored [out, in] row-major, the layout of the paper's
    projection V' = V W^T + b (Section 3.3, "Dense work across valid
    positions"); no biases:
        Wa, Wb: [c_z, c_s]   W1: [hidden, c_z]   W2: [c_z, hidden]
        Wo: [c_s, c_z]
  * bf16 values are carried as uint16 bit patterns plus their exact float64
    values; fp32 values as float32 arrays plus their float64 values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

WEIGHT_NAMES = ("Wa", "Wb", "W1", "W2", "Wo")


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a length regime, widths, dtype and depth."""
    name: str
    index: int
    lengths: Optional[tuple]      # fixed lengths, or None when drawn
    draw: Optional[tuple]         # ("uniform", lo, hi) or ("loguniform", lo, hi)
    B: int
    c_s: int
    c_z: int
    hidden: int
    dtype: str                    # "f32" or "bf16"
    blocks: int


# The five workloads, in order. Index i is also the seed of its generator.
WORKLOADS: List[Workload] = [
    Workload("tiny_fp32", 0, (7, 12, 5, 16), None, 4, 16, 8, 16, "f32", 1),
    Workload("one_block_bf16", 1, None, ("uniform", 64, 128), 8, 128, 64, 128, "bf16", 1),
    Workload("near_uniform_x4", 2, None, ("uniform", 230, 256), 16, 384, 128, 512, "bf16", 4),
    Workload("high_variation_x4", 3, None, ("loguniform", 16, 512), 16, 384, 128, 512, "bf16", 4),
    Workload("long_square_x4", 4, (1024, 768, 384, 96), None, 4, 384, 128, 512, "bf16", 4),
]


def workload(index_or_name) -> Workload:
    if isinstance(index_or_name, int):
        return WORKLOADS[index_or_name]
    for w in WORKLOADS:
        if w.name == index_or_name:
            return w
    raise KeyError(index_or_name)


# ---------------------------------------------------------------- dtype casts
def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns. Inputs here are finite.
    """
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    u32 = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Tensor:
    """A stored array: ``data`` is what goes to the device, ``f64`` its exact value."""
    data: np.ndarray
    f64: np.ndarray
    dtype: str


def store(x: np.ndarray, dtype: str) -> Tensor:
    """Cast drawn float64 values to the storage dtype: f64 -> f32 (-> bf16)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return Tensor(x32, x32.astype(np.float64), "f32")
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Tensor(bits, bf16_bits_to_f64(bits), "bf16")
    raise ValueError(dtype)


# ---------------------------------------------------------------- draws
def draw_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.lengths is not None:
        return np.asarray(w.lengths, dtype=np.int32)
    kind, lo, hi = w.draw
    if kind == "uniform":
        return rng.integers(lo, hi + 1, w.B).astype(np.int32)
    if kind == "loguniform":
        x = np.exp(rng.uniform(math.log(lo), math.log(hi), w.B))
        return np.clip(np.rint(x), lo, hi).astype(np.int32)
    raise ValueError(kind)


def draw_weights(rng: np.random.Generator, c_s: int, c_z: int, hidden: int,
                 dtype: str) -> dict:
    """One block's weights, N(0, 1/fan_in), drawn [in, out] then stored [out, in]."""
    shapes = {"Wa": (c_s, c_z), "Wb": (c_s, c_z), "W1": (c_z, hidden),
              "W2": (hidden, c_z), "Wo": (c_z, c_s)}
    out = {}
    for name in WEIGHT_NAMES:
        fan_in, fan_out = shapes[name]
        w = rng.standard_normal((fan_in, fan_out)) / math.sqrt(fan_in)
        out[name] = store(np.ascontiguousarray(w.T), dtype)
    return out


@dataclasses.dataclass
class Inputs:
    lengths: np.ndarray           # int32 [B]
    s: Tensor                     # [T, c_s]
    weights: List[dict]           # one dict of Tensors per block
    c_s: int
    c_z: int
    hidden: int
    dtype: str
    name: str = "custom"


def make_inputs(lengths: Sequence[int], c_s: int, c_z: int, hidden: int,
                dtype: str, blocks: int = 1, seed: int = 0,
                rng: Optional[np.random.Generator] = None,
                name: str = "custom") -> Inputs:
    """Singles ~ N(0, 1) and per-block weights ~ N(0, 1/fan_in), seeded."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32)
    T = int(lengths.astype(np.int64).sum())
    s = store(rng.standard_normal((T, c_s)), dtype)
    weights = [draw_weights(rng, c_s, c_z, hidden, dtype) for _ in range(blocks)]
    return Inputs(lengths, s, weights, c_s, c_z, hidden, dtype, name)


SWIGLU_NAMES = ("Wa", "Wb", "Wo", "ln_gamma", "ln_beta", "W_gate", "W_up", "W_down")


def draw_swiglu_weights(rng: np.random.Generator, c_s: int, c_z: int, hidden: int,
                        dtype: str) -> dict:
    """One block's parameters for the pre-normalised SwiGLU transition: the
    projections and the three products N(0, 1/fan_in), drawn [in, out] then
    stored [out, in] in `dtype`; the LayerNorm affine pair stored fp32,
    gamma ~ 1 + 0.2 N(0, 1) and beta ~ 0.1 N(0, 1) (away from the identity
    initialisation, so that both reach the results)."""
    shapes = {"Wa": (c_s, c_z), "Wb": (c_s, c_z), "Wo": (c_z, c_s), "W_gate": (c_z, hidden),
              "W_up": (c_z, hidden), "W_down": (hidden, c_z)}
    out = {}
    for name in SWIGLU_NAMES:
        if name == "ln_gamma":
            out[name] = store(1.0 + 0.2 * rng.standard_normal(c_z), "f32")
        elif name == "ln_beta":
            out[name] = store(0.1 * rng.standard_normal(c_z), "f32")
        else:
            fan_in, fan_out = shapes[name]
            w = rng.standard_normal((fan_in, fan_out)) / math.sqrt(fan_in)
            out[name] = store(np.ascontiguousarray(w.T), dtype)
    return out


def make_swiglu_inputs(lengths: Sequence[int], c_s: int, c_z: int, hidden: int, dtype: str,
                       blocks: int = 1, seed: int = 0) -> Inputs:
    """Singles ~ N(0, 1) and per-block SwiGLU-block parameters, seeded."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32)
    T = int(lengths.astype(np.int64).sum())
    s = store(rng.standard_normal((T, c_s)), dtype)
    weights = [draw_swiglu_weights(rng, c_s, c_z, hidden, dtype) for _ in range(blocks)]
    return Inputs(lengths, s, weights, c_s, c_z, hidden, dtype, "swiglu")


def workload_inputs(index_or_name, blocks: Optional[int] = None) -> Inputs:
    """The seeded inputs of a workload: lengths, then singles, then weights."""
    w = workload(index_or_name)
    rng = np.random.default_rng(w.index)
    lengths = draw_lengths(w, rng)
    return make_inputs(lengths, w.c_s, w.c_z, w.hidden, w.dtype,
                       blocks=w.blocks if blocks is None else blocks,
                       rng=rng, name=w.name)


def exact_inputs(lengths: Sequence[int], c_s: int, c_z: int, hidden: int,
                 dtype: str, seed: int = 0, blocks: int = 1,
                 nnz: int = 2) -> Inputs:
    """Inputs on which every intermediate of the block is a small integer.

    Singles are integers in [-2, 2]; each weight row holds at most ``nnz``
    entries drawn from {-1, +1} (the rest zero). With power-of-two lengths
    the column mean divides exactly, so both dtypes represent every stage
    without rounding.
    """
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32)
    T = int(lengths.astype(np.int64).sum())
    s = store(rng.integers(-2, 3, (T, c_s)).astype(np.float64), dtype)

    def sparse(out_dim, in_dim):
        w = np.zeros((out_dim, in_dim))
        for o in range(out_dim):
            cols = rng.choice(in_dim, size=min(nnz, in_dim), replace=False)
            w[o, cols] = rng.choice([-1.0, 1.0], size=cols.size)
        return store(w, dtype)

    weights = []
    for _ in range(blocks):
        weights.append({"Wa": sparse(c_z, c_s), "Wb": sparse(c_z, c_s),
                        "W1": sparse(hidden, c_z), "W2": sparse(c_z, hidden),
                        "Wo": sparse(c_s, c_z)})
    return Inputs(lengths, s, weights, c_s, c_z, hidden, dtype, "exact")


def random_pair_rows(lengths: Sequence[int], c_z: int, dtype: str,
                     seed: int = 0) -> Tensor:
    """A random packed pair state [sum N_i^2, c_z] (for stage-level tests)."""
    rng = np.random.default_rng(seed)
    cells = int((np.asarray(lengths, dtype=np.int64) ** 2).sum())
    return store(rng.standard_normal((cells, c_z)), dtype)


def random_rows(n: int, width: int, dtype: str, seed: int = 0,
                scale: float = 1.0) -> Tensor:
    rng = np.random.default_rng(seed)
    return store(scale * rng.standard_normal((n, width)), dtype)
