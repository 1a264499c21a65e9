#!/usr/bin/env python3
"""Benchmark of the packed single-pair-single block on one MI355X.

One step = the whole hot path on one batch: build the partition from host
lengths (offset scan, row splits), then every block of the workload
(projections, broadcast fused into the transition, column mean, output
projection). Inputs are resident in HBM before timing starts. The line also
carries the training step (forward, Equation 5 loss, backward) as "train".
Prints one JSON line; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import pair_inputs as pin  # noqa: E402

HEADLINE = "long_square_x4"
METRIC = "pair cells/sec per block (1 GPU) + HBM GB/s & MFMA util vs peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector/MFMA


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def dev(t: pin.Tensor, torch):
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(
            torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.data)).cuda()


class PackedRunner:
    """Preallocated buffers and one-step function for a workload."""

    def __init__(self, x: pin.Inputs, torch, nt):
        self.torch, self.nt, self.x = torch, nt, x
        self.lengths = torch.from_numpy(x.lengths.astype(np.int32)).pin_memory()
        T, cells, _, nbytes = nt.nt_partition_sizes(x.lengths)
        self.T, self.cells = T, cells
        self.part_buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        self.p = nt.nt_make_partition(self.lengths, buffer=self.part_buf)
        tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
        self.s0 = dev(x.s, torch)
        self.s = [torch.empty_like(self.s0), torch.empty_like(self.s0)]
        self.z = torch.empty((cells, x.c_z), dtype=tdt, device="cuda")
        self.ws = torch.empty(max(nt.nt_block_workspace_bytes(self.p, x.c_s, x.c_z, x.hidden, tdt),
                                  1), dtype=torch.uint8, device="cuda")
        self.w = [{k: dev(v, torch) for k, v in wk.items()} for wk in x.weights]
        # the blocks through one nt_pair_chain call instead of one call each
        self.chain = False
        self.chain_ws = None

    def use_chain(self):
        x, torch, nt = self.x, self.torch, self.nt
        tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
        self.chain_ws = self.torch.empty(max(nt.nt_chain_workspace_bytes(
            self.p, len(self.w), x.c_s, x.c_z, x.hidden, tdt), 1), dtype=torch.uint8,
            device="cuda")
        self.chain = True

    def step(self):
        nt = self.nt
        p = nt.nt_make_partition(self.lengths, buffer=self.part_buf)
        if self.chain:
            nt.nt_pair_chain(p, self.s0, self.w, s_out=self.s[1], z_out=self.z,
                             workspace=self.chain_ws)
            return self.s[1], self.z
        s_in = self.s0
        for k, w in enumerate(self.w):
            s_out = self.s[k % 2]
            nt.nt_pair_block(p, s_in, w, s_out=s_out, z_out=self.z, workspace=self.ws)
            s_in = s_out
        return s_in, self.z


class PerSampleRunner:
    """The matched-granularity control (DanLing NestedTensor, Section 4
    "Separating interface cost from execution strategy" and Appendix C.8,
    Table 7): the same kernels, issued once per sample instead of once per
    batch. Each sample gets its own one-sample partition and works on its
    contiguous slices of the packed singles and pair state."""

    def __init__(self, x: pin.Inputs, torch, nt, packed: PackedRunner):
        self.torch, self.nt, self.x, self.r = torch, nt, x, packed
        L = [int(n) for n in x.lengths]
        self.L = L
        self.eta = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
        self.o = np.concatenate([[0], np.cumsum(np.square(np.asarray(L, dtype=np.int64)))])
        self.lengths = [torch.tensor([n], dtype=torch.int32).pin_memory() for n in L]
        self.bufs = [torch.empty(max(nt.nt_partition_sizes([n])[3], 256), dtype=torch.uint8,
                                 device="cuda") for n in L]
        tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
        ws = max(nt.nt_block_workspace_bytes(nt.nt_make_partition([n]), x.c_s, x.c_z, x.hidden,
                                             tdt) for n in L)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")

    def step(self):
        nt, r = self.nt, self.r
        parts = [nt.nt_make_partition(self.lengths[i], buffer=self.bufs[i])
                 for i in range(len(self.L))]
        s_in = r.s0
        for k, w in enumerate(r.w):
            s_out = r.s[k % 2]
            for i, p in enumerate(parts):
                if self.L[i] == 0:
                    continue
                e0, e1 = int(self.eta[i]), int(self.eta[i + 1])
                o0, o1 = int(self.o[i]), int(self.o[i + 1])
                nt.nt_pair_block(p, s_in[e0:e1], w, s_out=s_out[e0:e1], z_out=r.z[o0:o1],
                                 workspace=self.ws)
            s_in = s_out
        return s_in, r.z


class TrainRunner:
    """Forward, Equation 5 loss and backward of the workload's blocks (the
    step the pages time: DanLing NestedTensor, Section 4 and Appendix A.1):
    every block keeps its input singles and returned pair state, the loss
    reads the last block's outputs, and the blocks' gradients run in reverse
    order. Buffers are preallocated; the partition is rebuilt each step."""

    def __init__(self, x: pin.Inputs, torch, nt, packed: PackedRunner):
        self.torch, self.nt, self.x, self.r = torch, nt, x, packed
        tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
        nb = len(x.weights)
        self.s = [packed.s0] + [torch.empty_like(packed.s0) for _ in range(nb)]
        self.z = [torch.empty((packed.cells, x.c_z), dtype=tdt, device="cuda")
                  for _ in range(nb)]
        self.g = [torch.empty((packed.T, x.c_s), dtype=torch.float32, device="cuda")
                  for _ in range(2)]
        self.grads = [{k: torch.empty(v.shape, dtype=torch.float32, device="cuda")
                       for k, v in w.items()} for w in packed.w]
        self.bws = torch.empty(max(nt.nt_block_backward_workspace_bytes(
            packed.p, x.c_s, x.c_z, x.hidden, tdt), 1), dtype=torch.uint8, device="cuda")
        self.lws = torch.empty(nt.nt_loss_workspace_bytes(packed.p), dtype=torch.uint8,
                               device="cuda")

    def step(self):
        nt, r = self.nt, self.r
        p = nt.nt_make_partition(r.lengths, buffer=r.part_buf)
        for k, w in enumerate(r.w):
            nt.nt_pair_block(p, self.s[k], w, s_out=self.s[k + 1], z_out=self.z[k],
                             workspace=r.ws)
        loss, g, g_pz = nt.nt_pair_loss_eq5(p, self.s[-1], self.z[-1], workspace=self.lws)
        for k in range(len(r.w) - 1, -1, -1):
            out = self.g[k % 2]
            nt.nt_pair_block_backward(p, self.s[k], self.z[k], r.w[k], g,
                                      g_pz if k == len(r.w) - 1 else None, g_s_in=out,
                                      grads=self.grads[k], workspace=self.bws)
            g = out
        return loss, g


class SwigluTrainRunner:
    """The same training step with the paper's own transition (the
    pre-normalised SwiGLU of expansion four, Equation 1 with h o LN;
    Appendix A.1; Table 1's program): every block is nt_pair_block_ex with
    seeded SwiGLU-block weights of the workload's widths, then Equation 5
    and nt_pair_block_backward_ex in reverse order."""

    def __init__(self, x: pin.Inputs, torch, nt, packed: PackedRunner):
        self.torch, self.nt, self.r = torch, nt, packed
        rng = np.random.default_rng(78)
        nb = len(x.weights)
        self.w = [{k: dev(v, torch) for k, v in
                   pin.draw_swiglu_weights(rng, x.c_s, x.c_z, x.hidden, x.dtype).items()}
                  for _ in range(nb)]
        tdt = torch.bfloat16
        self.s = [packed.s0] + [torch.empty_like(packed.s0) for _ in range(nb)]
        self.z = [torch.empty((packed.cells, x.c_z), dtype=tdt, device="cuda") for _ in range(nb)]
        self.g = [torch.empty((packed.T, x.c_s), dtype=torch.float32, device="cuda")
                  for _ in range(2)]
        self.grads = [{k: torch.empty(v.shape, dtype=torch.float32, device="cuda")
                       for k, v in w.items()} for w in self.w]
        kind = nt.NT_TRANSITION_LN_SWIGLU
        self.bws = torch.empty(max(nt.nt_block_backward_ex_workspace_bytes(
            packed.p, kind, x.c_s, x.c_z, x.hidden, tdt), 1), dtype=torch.uint8, device="cuda")
        self.lws = torch.empty(nt.nt_loss_workspace_bytes(packed.p), dtype=torch.uint8,
                               device="cuda")

    def forward(self):
        nt, r = self.nt, self.r
        p = nt.nt_make_partition(r.lengths, buffer=r.part_buf)
        for k, w in enumerate(self.w):
            nt.nt_pair_block_ex(p, self.s[k], w, s_out=self.s[k + 1], z_out=self.z[k],
                                workspace=r.ws)
        return p

    def step(self):
        nt = self.nt
        p = self.forward()
        loss, g, g_pz = nt.nt_pair_loss_eq5(p, self.s[-1], self.z[-1], workspace=self.lws)
        for k in range(len(self.w) - 1, -1, -1):
            out = self.g[k % 2]
            nt.nt_pair_block_backward_ex(p, self.s[k], self.z[k], self.w[k], g,
                                         g_pz if k == len(self.w) - 1 else None, g_s_in=out,
                                         grads=self.grads[k], workspace=self.bws)
            g = out
        return loss, g


def backward_rooflines(r: PackedRunner, reps: int) -> dict:
    """The transition's gradient on block 0's pair state (matrix-core act
    kernel plus the two weight-gradient contractions, one call), against
    the bf16 MFMA peak: five products of 2 c_z h flop per cell."""
    torch, nt, x = r.torch, r.nt, r.x
    if x.dtype != "bf16":
        return {}
    w = r.w[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    G = torch.randn((r.cells, x.c_z), device="cuda", generator=g) / 64
    g_z = torch.empty_like(G)
    dW1 = torch.empty((x.hidden, x.c_z), device="cuda")
    dW2 = torch.empty((x.c_z, x.hidden), device="cuda")
    ws = torch.empty(nt.nt_transition_backward_workspace_bytes(r.p, x.c_z, x.hidden,
                                                               torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    t = time_kernel(lambda: nt.nt_pair_transition_backward(r.p, r.z, G, w["W1"], w["W2"],
                                                           g_z=g_z, dW1=dW1, dW2=dW2,
                                                           workspace=ws), reps, torch)
    flops = 10.0 * x.c_z * x.hidden * r.cells
    return {"kernel": "k_transition_bwd + k_wgrad_rc (transition gradient, one call)",
            "bound": "mfma", "ms": t * 1e3, "achieved": flops / t / 1e12,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "flop_per_launch": flops,
            "frac": flops / t / 1e12 / PEAK_BF16_TFLOPS}


def rectangular(x: pin.Inputs, args, torch, nt) -> dict:
    """The rectangular variant (Appendix A.1) on the workload's shapes: pair
    rows from the workload's singles (lengths N_i), pair columns from a second
    set of singles whose lengths are the same lengths in reverse order (M_i),
    the same four blocks; cells/s per block of the N_i x M_i pair state."""
    rows = [int(n) for n in x.lengths]
    cols = rows[::-1]
    tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    s_rows = dev(x.s, torch)
    s_cols = torch.randn(sum(cols), x.c_s, device="cuda", generator=g).to(tdt)
    lengths_r = torch.tensor(rows, dtype=torch.int32).pin_memory()
    lengths_c = torch.tensor(cols, dtype=torch.int32).pin_memory()
    _, _, cells, nbytes = nt.nt_partition_sizes_rect(rows, cols)
    buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    p = nt.nt_make_partition_rect(rows, cols, buffer=buf)
    ws = torch.empty(max(nt.nt_block_workspace_bytes(p, x.c_s, x.c_z, x.hidden, tdt), 1),
                     dtype=torch.uint8, device="cuda")
    z = torch.empty((cells, x.c_z), dtype=tdt, device="cuda")
    outs = [torch.empty_like(s_rows), torch.empty_like(s_rows)]
    weights = [{k: dev(v, torch) for k, v in wk.items()} for wk in x.weights]

    def step():
        q = nt.nt_make_partition_rect(rows, cols, buffer=buf)
        s_in = s_rows
        for k, w in enumerate(weights):
            s_out = outs[k % 2]
            nt.nt_pair_block_rect(q, s_in, s_cols, w, s_out=s_out, z_out=z, workspace=ws)
            s_in = s_out

    t = time_steps(step, args.steps, args.warmup, torch)
    log(f"rectangular (M = reversed N): {cells} cells, {t * 1e3:.3f} ms/step -> "
        f"{cells * len(weights) / t:.4g} cells/s per block")
    return {"rows": rows, "cols": cols, "cells": cells, "blocks": len(weights),
            "ms_per_step": t * 1e3, "value": cells * len(weights) / t,
            "unit": "pair cells/s per block"}


def non_leading(x: pin.Inputs, args, torch, nt, S: int = 3) -> dict:
    """The non-leading variant (Appendix A.1, S = 3): the workload's lengths
    and widths with a static axis of S slices in every single row and pair
    cell, the same four blocks; forward and the training step (forward,
    Equation 5 with S, backward). Cells/s per block counts pair cells (each
    holding S slices)."""
    tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    lengths = torch.from_numpy(x.lengths.astype(np.int32)).pin_memory()
    T, cells, _, nbytes = nt.nt_partition_sizes(x.lengths)
    buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    p = nt.nt_make_partition(lengths, buffer=buf)
    s0 = torch.randn(T, S * x.c_s, device="cuda", generator=g).to(tdt)
    weights = [{k: dev(v, torch) for k, v in wk.items()} for wk in x.weights]
    nb = len(weights)
    s = [s0] + [torch.empty_like(s0) for _ in range(nb)]
    z = [torch.empty((cells, S * x.c_z), dtype=tdt, device="cuda") for _ in range(nb)]
    ws = torch.empty(max(nt.nt_block_nl_workspace_bytes(p, S, x.c_s, x.c_z, x.hidden, tdt), 1),
                     dtype=torch.uint8, device="cuda")
    bws = torch.empty(max(nt.nt_block_backward_nl_workspace_bytes(p, S, x.c_s, x.c_z, x.hidden,
                                                                  tdt), 1),
                      dtype=torch.uint8, device="cuda")
    gbuf = [torch.empty((T, S * x.c_s), dtype=torch.float32, device="cuda") for _ in range(2)]
    grads = [{k: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in w.items()}
             for w in weights]

    def forward():
        q = nt.nt_make_partition(lengths, buffer=buf)
        for k, w in enumerate(weights):
            nt.nt_pair_block_nl(q, s[k], w, S, s_out=s[k + 1], z_out=z[k], workspace=ws)
        return q

    def train():
        q = forward()
        loss, gx, gp = nt.nt_pair_loss_eq5(q, s[-1], z[-1], S=S)
        gcur = gx
        for k in range(nb - 1, -1, -1):
            out = gbuf[k % 2]
            nt.nt_pair_block_backward_nl(q, s[k], z[k], weights[k], S, gcur,
                                         gp if k == nb - 1 else None, g_s_in=out,
                                         grads=grads[k], workspace=bws)
            gcur = out

    t_f = time_steps(forward, args.steps, args.warmup, torch)
    t_t = time_steps(train, max(3, args.steps // 2), 2, torch)
    log(f"non-leading S={S}: forward {t_f * 1e3:.3f} ms/step "
        f"({cells * nb / t_f:.4g} cells/s per block), train step {t_t * 1e3:.3f} ms")
    return {"S": S, "cells": cells, "blocks": nb, "forward_ms_per_step": t_f * 1e3,
            "forward_value": cells * nb / t_f, "train_ms_per_step": t_t * 1e3,
            "train_value": cells * nb / t_t, "unit": "pair cells/s per block (S slices per cell)",
            "path": "the broadcast fused into the weight-stationary transition over the S "
                    "slices of every cell (k_transition_ws), then the column mean over rows of "
                    "S c_z values"}


def granularity(x: pin.Inputs, r: PackedRunner, t_seg: float, args, torch, nt) -> dict:
    """Per-sample launches against the segmented launch on the same kernels:
    the granularity gain is per-sample time over segmented time."""
    ps = PerSampleRunner(x, torch, nt, r)
    t_ps = time_steps(ps.step, max(3, args.steps // 2), 2, torch)
    log(f"per-sample launches {t_ps * 1e3:.3f} ms vs segmented {t_seg * 1e3:.3f} ms "
        f"-> {t_ps / t_seg:.2f}x")
    return {"segmented_ms_per_step": t_seg * 1e3, "per_sample_ms_per_step": t_ps * 1e3,
            "gain": t_ps / t_seg, "launches_per_step_per_sample": len(x.weights) * 4 + 1,
            "samples": len(x.lengths)}


def hbm_ceiling(torch) -> dict:
    """Practical HBM rates on this device, as a reference beside the spec
    peak (the kernels are graded against the spec): a torch device copy of
    1 GiB each way and a torch fill of 512 MiB, HIP-event timed."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = time_kernel(lambda: dst.copy_(src), 20, torch)
    half = dst[: n // 2]
    t_fill = time_kernel(lambda: half.fill_(2.0), 20, torch)
    del src, dst, half
    torch.cuda.empty_cache()
    copy_gbs = 2 * n * 4 / t_copy / 1e9
    fill_gbs = n // 2 * 4 / t_fill / 1e9
    return {"copy_GBps": copy_gbs, "copy_frac": copy_gbs / PEAK_HBM_GBS,
            "fill_GBps": fill_gbs, "fill_frac": fill_gbs / PEAK_HBM_GBS,
            "impl": "torch copy_ (1 GiB read + 1 GiB written) and fill_ (512 MiB written)"}


def step_spread(fn, steps: int, torch) -> dict:
    """Median and minimum of single steps, from HIP events recorded between
    `steps` further back-to-back steps (after the timed region, which stays
    bracketed by synchronisations only)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for k in range(steps):
        fn()
        ev[k + 1].record()
    ev[-1].synchronize()
    d = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(steps))
    return {"median": d[len(d) // 2], "min": d[0], "max": d[-1], "steps": steps}


def settle(fn, ms: float, torch) -> int:
    """Repeat fn for `ms` milliseconds of wall time (untimed), so that the
    timed steps and kernel timings see the clocks a GPU holds under sustained
    load: over the first few hundred milliseconds of work they are still
    rising, and a kernel runs up to 20% slower. Returns the number of calls."""
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    return n


def time_steps(fn, steps: int, warmup: int, torch) -> float:
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_kernel(fn, reps: int, torch) -> float:
    """Average duration (s) of fn's launches, from HIP events on the current
    stream (the stream the library launches on)."""
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / 1e3 / reps


def time_kernel_in_steps(fn, step, reps: int, torch) -> float:
    """Average duration (s) of fn's launches when each is followed by a whole
    step, as the kernel runs inside the hot path, from HIP events recorded on
    the current stream right before and after it. Back to back, an MFMA-bound
    kernel draws power without pause and the clocks sag after a few launches;
    in steps the memory-bound kernels between its launches leave headroom."""
    for _ in range(5):
        fn()
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    for k in range(reps):
        ev[2 * k].record()
        fn()
        ev[2 * k + 1].record()
        step()
    ev[-1].synchronize()
    return sum(ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(reps)) / 1e3 / reps


def transition_kernel_id(c_z: int, hidden: int, dtype: str) -> str:
    """The kernel the library launches for the fused broadcast + transition
    (batches of fewer than 2^22 single rows)."""
    if dtype == "bf16" and c_z == 128 and hidden == 512:
        return "k_transition_ws"
    if dtype == "bf16" and (c_z, hidden) == (64, 128):
        return "k_transition_p32"
    return "fused"


def transition_kernel_label(c_z: int, hidden: int, dtype: str) -> str:
    """The kernel the library launches for the fused broadcast + transition."""
    kid = transition_kernel_id(c_z, hidden, dtype)
    if kid == "k_transition_ws":
        return "k_transition_ws (fused broadcast, weights resident in registers)"
    if kid == "k_transition_p32":
        return "k_transition_p32 (fused broadcast prologue)"
    return "fused broadcast + transition"


def kernel_rooflines(r: PackedRunner, reps: int):
    """Per-kernel durations on block 0's data: the fused broadcast+transition
    (the kernel the block launches), the standalone broadcast and the column
    mean, each against its roofline."""
    torch, nt, x = r.torch, r.nt, r.x
    w = r.w[0]
    # a and b as the block's projections produce them, fp32 (harness inputs only)
    s32 = r.s0.float()
    a32 = (s32 @ w["Wa"].float().t().contiguous()).contiguous()
    b32 = (s32 @ w["Wb"].float().t().contiguous()).contiguous()
    a, b = a32.to(r.s0.dtype), b32.to(r.s0.dtype)
    es = 2 if x.dtype == "bf16" else 4
    T, cells, cz, hd = r.T, r.cells, x.c_z, x.hidden
    m = torch.empty((T, cz), dtype=torch.float32, device="cuda")
    zt = torch.empty_like(r.z)
    out = {}

    def fused():
        nt.nt_pair_broadcast_transition(r.p, a32, b32, w["W1"], w["W2"], z_out=r.z)
    t_b2b = time_kernel(fused, reps, torch)
    t = time_kernel_in_steps(fused, r.step, reps, torch)
    flops = 4.0 * cz * hd * cells
    nbytes = cells * cz * es + 2 * T * cz * 4 + 2 * hd * cz * es
    peak_f = PEAK_BF16_TFLOPS if x.dtype == "bf16" else PEAK_F32_TFLOPS
    t_f, t_b = flops / (peak_f * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)
    label = transition_kernel_label(cz, hd, x.dtype)
    if t_f >= t_b:
        out["transition"] = {"kernel": label,
                             "bound": "mfma", "ms": t * 1e3, "achieved": flops / t / 1e12,
                             "peak": peak_f, "unit": "TFLOP/s", "flop_per_launch": flops,
                             "bytes_per_launch": nbytes, "timing": "in steps",
                             "back_to_back_ms": t_b2b * 1e3}
    else:
        out["transition"] = {"kernel": label,
                             "bound": "hbm", "ms": t * 1e3, "achieved": nbytes / t / 1e9,
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "flop_per_launch": flops,
                             "bytes_per_launch": nbytes, "timing": "in steps",
                             "back_to_back_ms": t_b2b * 1e3}
    t = time_kernel(lambda: nt.nt_pair_broadcast(r.p, a, b, z=zt), reps, torch)
    nbytes = cells * cz * es + 2 * T * cz * es
    # the stage's kernel: tiles of one sample for at most 256 samples
    bkern = "k_broadcast_tiled" if len(r.lengths) <= 256 else "k_broadcast"
    out["broadcast"] = {"kernel": bkern, "bound": "hbm", "ms": t * 1e3,
                        "achieved": nbytes / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "bytes_per_launch": nbytes}
    t = time_kernel(lambda: nt.nt_pair_reduce(r.p, zt, m=m), reps, torch)
    nbytes = cells * cz * es + T * cz * 4
    out["reduce"] = {"kernel": "k_reduce_pow2", "bound": "hbm", "ms": t * 1e3,
                     "achieved": nbytes / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "bytes_per_launch": nbytes}
    for v in out.values():
        v["frac"] = v["achieved"] / v["peak"]
    return out


def swiglu_roofline(r: PackedRunner, reps: int) -> dict:
    """The paper's pre-normalised SwiGLU transition (expansion four) on the
    workload's pair state: 6 c_z h flop per cell (gate, value and down
    products), against the bf16 MFMA peak."""
    torch, nt, x = r.torch, r.nt, r.x
    cz, hd = x.c_z, x.hidden
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    gamma = 1.0 + 0.2 * torch.randn(cz, device="cuda", generator=g)
    beta = 0.1 * torch.randn(cz, device="cuda", generator=g)
    Wg = (torch.randn(hd, cz, device="cuda", generator=g) / cz ** 0.5).to(torch.bfloat16)
    Wu = (torch.randn(hd, cz, device="cuda", generator=g) / cz ** 0.5).to(torch.bfloat16)
    Wd = (torch.randn(cz, hd, device="cuda", generator=g) / hd ** 0.5).to(torch.bfloat16)
    out = torch.empty_like(r.z)
    t = time_kernel(lambda: nt.nt_pair_transition_swiglu(r.p, r.z, gamma, beta, Wg, Wu, Wd,
                                                         z_out=out), reps, torch)
    flops = 6.0 * cz * hd * r.cells
    return {"kernel": "k_swiglu32 (LN + SwiGLU, expansion four; unfused stage)", "bound": "mfma",
            "ms": t * 1e3, "achieved": flops / t / 1e12, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "flop_per_launch": flops,
            "frac": flops / t / 1e12 / PEAK_BF16_TFLOPS}


def swiglu_block(r: PackedRunner, reps: int) -> dict:
    """The paper's own block end to end (Equation 1 with h o LN; App. A.1):
    nt_pair_block_ex with the pre-normalised SwiGLU transition on the
    workload's singles, seeded SwiGLU-block weights of its widths. One
    block: projections, the fused broadcast + LN + SwiGLU + residual
    (k_swiglu32), the column mean and the output projection. `frac` counts
    only the transition's 6 c_z h flop per cell against the whole block's
    time, a lower bound of the fused kernel's own fraction."""
    torch, nt, x = r.torch, r.nt, r.x
    w = pin.draw_swiglu_weights(np.random.default_rng(77), x.c_s, x.c_z, x.hidden, x.dtype)
    params = {k: dev(v, torch) for k, v in w.items()}
    s_out = torch.empty_like(r.s0)
    z_out = torch.empty_like(r.z)
    ws = torch.empty(max(nt.nt_block_workspace_bytes(r.p, x.c_s, x.c_z, x.hidden, torch.bfloat16),
                         1), dtype=torch.uint8, device="cuda")
    t = time_kernel(lambda: nt.nt_pair_block_ex(r.p, r.s0, params, s_out=s_out, z_out=z_out,
                                                workspace=ws), reps, torch)
    flops = 6.0 * x.c_z * x.hidden * r.cells
    return {"kernel": "nt_pair_block_ex, SwiGLU kind (k_swiglu32 fused, with the block's "
                      "projections and column mean)", "bound": "mfma",
            "ms": t * 1e3, "cells_per_s": r.cells / t, "achieved": flops / t / 1e12,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "flop_per_launch": flops,
            "frac": flops / t / 1e12 / PEAK_BF16_TFLOPS}


def counters_for(kernel_key: str) -> dict:
    """The committed rocprofv3 counter results of a kernel (HBM bytes per
    launch, matrix-pipe busy fraction), if they were taken on the current
    kernel source; otherwise an empty dict."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    entry = data.get(kernel_key)
    if not entry or entry.get("kernel") != kernel_key.split(":")[0]:
        return {}
    src = os.path.join(ROOT, "padding_free_pair_amd", "csrc", entry["source"])
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if digest != entry.get("source_sha256"):
        return {}
    return entry


def traffic_for(kernel_key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; otherwise None."""
    return counters_for(kernel_key).get("bytes_per_launch")


def padded_same_kernels(x: pin.Inputs, steps: int, warmup: int, torch, nt) -> float:
    """Step time of this library's own kernels over the B x N_max^2 envelope:
    every sample padded to N_max with zero singles, the same weights. It
    separates the cost of padding from the choice of kernels. It is a timing
    baseline only: the kernels have no validity mask, so the padded columns
    enter the mean."""
    L = x.lengths.astype(np.int64)
    B, nmax = len(L), int(L.max())
    eta = np.concatenate([[0], np.cumsum(L)])
    s64 = np.zeros((B * nmax, x.c_s))
    for i in range(B):
        s64[i * nmax: i * nmax + L[i]] = x.s.f64[eta[i]: eta[i + 1]]
    env = dataclasses.replace(x, lengths=np.full(B, nmax, dtype=np.int32),
                              s=pin.store(s64, x.dtype))
    r = PackedRunner(env, torch, nt)
    t = time_steps(r.step, steps, warmup, torch)
    del r
    torch.cuda.empty_cache()
    return t


class PaddedEnvelope:
    """The padded comparator (DanLing NestedTensor, Section 4.1
    "Measurement": padding is the baseline; Table 2's caption: padding runs
    native PyTorch kernels): the same blocks over the B x N_max^2 envelope
    with PyTorch ops on zero-padded singles, a validity mask over the
    columns and the mean over valid columns only. Its rounding points are
    the packed path's, so both meet the same bound against the oracle: fp32
    projections, the pair state rounded to the storage type as the MLP's
    operand, the residual added in fp32 and rounded once, an fp32 mean and
    output projection. It is the comparator of the packed path, not part of
    it, and it runs on any torch device."""

    def __init__(self, x: pin.Inputs, torch, device="cuda"):
        self.torch, self.x = torch, x
        L = x.lengths.astype(np.int64)
        self.B, self.N = len(L), int(L.max()) if len(L) else 0
        self.tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
        self.fp32_out = torch.device(device).type == "cuda"
        B, N = self.B, self.N
        s = dev(x.s, torch).to(device)
        eta = np.concatenate([[0], np.cumsum(L)])
        self.S0 = torch.zeros((B, N, x.c_s), dtype=self.tdt, device=device)
        self.colmask = torch.zeros((B, 1, N, 1), dtype=self.tdt, device=device)
        for i in range(B):
            self.S0[i, :L[i]] = s[eta[i]:eta[i + 1]]
            self.colmask[i, :, :L[i]] = 1
        # every row of an empty sample is padding: its count only avoids 0/0
        self.cnt = torch.from_numpy(np.maximum(L, 1).astype(np.float32)).to(device)[:, None, None]
        self.W = []
        for wk in x.weights:
            w = {k: dev(v, torch).to(device).t().contiguous() for k, v in wk.items()}  # [in, out]
            for k in ("Wa", "Wb", "Wo"):
                w[k] = w[k].float()
            self.W.append(w)

    def _add_product(self, Z, H, W2):
        """Z + H W2 in fp32 (the packed path's residual). On a GPU the product
        of the bf16 operands is written in fp32 by the GEMM itself (torch's
        out_dtype); where torch has no such kernel the product is rounded to
        the storage type first, one rounding more than the packed path."""
        torch = self.torch
        if self.fp32_out and H.dtype == torch.bfloat16:
            try:
                return torch.addmm(Z, H, W2, out_dtype=torch.float32)
            except (RuntimeError, TypeError, NotImplementedError):
                self.fp32_out = False
        Z += (H @ W2).float()
        return Z

    def step(self):
        """One pass of every block; returns the last block's singles
        [B, N_max, c_s] and pair state [B * N_max^2, c_z] (invalid columns
        zeroed by the mask)."""
        torch, x, B, N = self.torch, self.x, self.B, self.N
        S, P = self.S0, None
        for w in self.W:
            S2 = S.reshape(-1, x.c_s).float()
            U = (S2 @ w["Wa"]).view(B, N, 1, x.c_z)
            V = (S2 @ w["Wb"]).view(B, 1, N, x.c_z)
            Z = (U + V).view(-1, x.c_z)                      # fp32 envelope
            H = torch.relu_(Z.to(self.tdt) @ w["W1"])
            Z = self._add_product(Z, H, w["W2"])
            del H
            P = Z.to(self.tdt)
            del Z
            P4 = P.view(B, N, N, x.c_z)
            P4.mul_(self.colmask)                            # mask invalid columns in place
            M = P4.sum(dim=2, dtype=torch.float32) / self.cnt
            S = (S2 + M.view(-1, x.c_z) @ w["Wo"]).to(self.tdt).view(B, N, x.c_s)
        return S, P

    def valid(self, S, P):
        """The valid rows of S and cells of P in packed order (eta and o)."""
        torch = self.torch
        L = self.x.lengths.astype(np.int64)
        rows = [S[i, :n] for i, n in enumerate(L)]
        P4 = P.view(self.B, self.N, self.N, -1)
        cells = [P4[i, :n, :n].reshape(-1, P.shape[-1]) for i, n in enumerate(L)]
        return torch.cat(rows), torch.cat(cells)


def padded_report(x: pin.Inputs, t_step: float, packed_peak: int, cells: int, args, torch,
                  nt) -> dict:
    """The padded comparator beside a packed measurement: step time, peak
    allocated bytes and the ratios S_m = T_pad / T and E_m = M_pad / M
    (DanLing NestedTensor, Section 4.1 "Measurement"), the pair occupancy
    rho_pair = sum N_i^2 / (B N_max^2), and this library's own block over
    the envelope (timing only), which separates the cost of padding from the
    choice of kernels."""
    env = int(x.lengths.max()) ** 2 * len(x.lengths)
    log(f"padded envelope baseline {x.name}")
    t_pad, pad_peak, fp32_out = padded_baseline(x, max(3, args.steps // 4), 2, torch)
    t_env = padded_same_kernels(x, args.steps, args.warmup, torch, nt)
    log(f"padded {t_pad * 1e3:.3f} ms/step ({t_pad / t_step:.2f}x); this library's kernels over "
        f"the envelope: {t_env * 1e3:.3f} ms/step ({t_env / t_step:.2f}x)")
    return {"ms_per_step": t_pad * 1e3, "speedup": t_pad / t_step, "envelope_cells": env,
            "rho_pair": cells / env, "peak_bytes_padded": pad_peak,
            "peak_bytes_packed": packed_peak, "memory_efficiency": pad_peak / max(packed_peak, 1),
            "impl": "PyTorch ops over B x N_max^2: fp32 projections, bf16 MLP products, fp32 "
                    "residual and masked mean (the packed path's rounding points)",
            "second_product_fp32_output": fp32_out,
            "same_kernels": {"ms_per_step": t_env * 1e3, "speedup": t_env / t_step,
                             "impl": "this library's block over every sample padded to N_max "
                                     "(timing only: no validity mask)"}}


def padded_baseline(x: pin.Inputs, steps: int, warmup: int, torch):
    """Step time and peak allocated bytes of the padded comparator."""
    env = PaddedEnvelope(x, torch)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    t = time_steps(env.step, steps, warmup, torch)
    peak = torch.cuda.max_memory_allocated() - base
    fp32_out = env.fp32_out
    del env
    torch.cuda.empty_cache()
    return t, peak, fp32_out


def host_threads() -> int:
    """Threads the oracle may use on this host: OMP_NUM_THREADS when the
    environment sets it (GPU hosts give each GPU its share of cores that
    way), otherwise the cores this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def oracle_rate(x: pin.Inputs, min_seconds: float, threads: int) -> dict:
    """The float64 oracle (oracle.block, as it stands) timed on this host
    with its BLAS limited to `threads`: the workload's blocks in order, each
    over its samples in batch order, one oracle.block call per sample (the
    block is sample-local, so this is the batch's arithmetic), until every
    block is done or at least min_seconds have passed. Returns pair cells/s
    per block over the sample-blocks timed."""
    import oracle
    from threadpoolctl import threadpool_limits
    L = [int(n) for n in x.lengths]
    eta = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    s = x.s.f64
    ws = [{k: v.f64 for k, v in wk.items()} for wk in x.weights]
    cells = units = 0
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        dt = 0.0
        for w in ws:
            for i, n in enumerate(L):
                oracle.block([n], s[eta[i]:eta[i + 1]], w)
                cells += n * n
                units += 1
                dt = time.perf_counter() - t0
                if dt >= min_seconds:
                    break
            if dt >= min_seconds:
                break
    total = len(ws) * len(L)
    return {"value": cells / dt, "unit": "pair cells/s per block", "cores": threads,
            "kind": "oracle", "seconds": dt,
            "sample": f"{units} of the {total} sample-blocks of {x.name} ({cells} cells), "
                      f"in order, one float64 oracle.block call each"}


def cpu_baseline(x: pin.Inputs, min_seconds: float = 12.0) -> dict:
    """The headline workload's oracle rate on the host's thread share, then
    the protocol's companions: the same on every other workload (a few
    seconds each), and one thread on the three smallest workloads."""
    threads = host_threads()
    out = oracle_rate(x, min_seconds, threads)
    out["host_cpus"] = len(os.sched_getaffinity(0))
    out["thread_env"] = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS",
                                                         "OPENBLAS_NUM_THREADS")}
    regimes, one = {}, {}
    for w in pin.WORKLOADS:
        xo = x if w.name == x.name else pin.workload_inputs(w.index)
        if w.name != x.name:
            regimes[w.name] = oracle_rate(xo, 3.0, threads)
        if w.index <= 2:
            one[w.name] = oracle_rate(xo, 4.0, 1)
    out["regimes"] = regimes
    out["one_thread"] = one
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--kernel-reps", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="untimed steps for this long before the warm-up steps, until the "
                         "GPU clocks have settled under load")
    ap.add_argument("--quick", action="store_true",
                    help="timed steps and kernel timings only (for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chain", action="store_true",
                    help="run each step's blocks through one nt_pair_chain call")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the packed block is sample-local and is not sharded here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import padding_free_pair_amd as nt
    nt._native.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_reference:
        # a plain copy kernel of known size: 1 GiB read + 1 GiB written per launch
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        t = time_kernel(lambda: dst.copy_(src), 5, torch)
        print(json.dumps({"copy_bytes_each_way": n * 4, "ms": t * 1e3,
                          "GB/s (read+write)": 2 * n * 4 / t / 1e9}))
        return

    w = pin.workload(args.workload)
    x = pin.workload_inputs(w.index)
    log(f"workload {w.name}: B={w.B} cells={int((x.lengths.astype(np.int64) ** 2).sum())} "
        f"blocks={w.blocks}")
    r = PackedRunner(x, torch, nt)
    if args.chain:
        r.use_chain()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_mem = torch.cuda.memory_allocated()
    settle_calls = settle(r.step, args.settle_ms, torch)
    t_step = time_steps(r.step, args.steps, args.warmup, torch)
    packed_peak = torch.cuda.max_memory_allocated() - base_mem + sum(
        t.numel() * t.element_size() for t in (r.z, r.ws, r.part_buf, r.s[0], r.s[1], r.s0))
    value = r.cells * w.blocks / t_step
    log(f"step {t_step * 1e3:.3f} ms -> {value:.4g} cells/s per block")
    spread = step_spread(r.step, args.steps, torch)

    kern = kernel_rooflines(r, args.kernel_reps)
    for k, v in kern.items():
        if "back_to_back_ms" in v:
            log(f"kernel {k} back to back: {v['back_to_back_ms'] * 1e3:.1f} us")
        log(f"kernel {k}: {v['ms'] * 1e3:.1f} us, {v['achieved']:.1f} {v['unit']} "
            f"({100 * v['frac']:.1f}% of peak)")
    if x.dtype == "bf16" and x.c_z in (64, 128) and x.hidden % 32 == 0:
        kern["swiglu_transition"] = swiglu_roofline(r, args.kernel_reps)
        v = kern["swiglu_transition"]
        log(f"kernel swiglu_transition: {v['ms'] * 1e3:.1f} us, {v['achieved']:.1f} TFLOP/s "
            f"({100 * v['frac']:.1f}% of peak)")
        if x.c_z == 128 and x.hidden % 64 == 0:
            kern["swiglu_block"] = swiglu_block(r, args.kernel_reps)
            v = kern["swiglu_block"]
            log(f"swiglu block (paper's transition, fused): {v['ms'] * 1e3:.1f} us per block, "
                f"{v['cells_per_s']:.4g} cells/s; transition flop {100 * v['frac']:.1f}% of peak")
    if x.dtype == "bf16":
        kern["transition_backward"] = backward_rooflines(r, max(10, args.kernel_reps // 5))
        v = kern["transition_backward"]
        log(f"kernel transition_backward: {v['ms'] * 1e3:.1f} us, {v['achieved']:.1f} TFLOP/s "
            f"({100 * v['frac']:.1f}% of peak)")
    tr = TrainRunner(x, torch, nt, r)
    t_train = time_steps(tr.step, args.steps, args.warmup, torch)
    train = {"value": r.cells * w.blocks / t_train, "unit": "pair cells/s per block",
             "ms_per_step": t_train * 1e3, "forward_ms": t_step * 1e3,
             "step": "forward of every block, Equation 5 loss, backward of every block"}
    log(f"train step {t_train * 1e3:.3f} ms -> {train['value']:.4g} cells/s per block")
    del tr
    torch.cuda.empty_cache()
    swiglu_train = None
    if x.dtype == "bf16" and x.c_z == 128 and x.hidden % 64 == 0:
        sr = SwigluTrainRunner(x, torch, nt, r)
        t_sf = time_steps(sr.forward, args.steps, args.warmup, torch)
        t_st = time_steps(sr.step, max(2, args.steps // 4), 2, torch)
        swiglu_train = {"value": r.cells * w.blocks / t_st, "unit": "pair cells/s per block",
                        "ms_per_step": t_st * 1e3, "forward_ms": t_sf * 1e3,
                        "step": "the paper's block (pre-normalised SwiGLU transition): forward "
                                "of every block, Equation 5 loss, backward of every block"}
        log(f"swiglu train step {t_st * 1e3:.3f} ms (forward {t_sf * 1e3:.3f} ms) -> "
            f"{swiglu_train['value']:.4g} cells/s per block")
        del sr
        torch.cuda.empty_cache()
    dom = kern["transition"]
    roofline = {"bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
                "unit": dom["unit"], "frac": dom["frac"],
                "traffic": traffic_for(f"{transition_kernel_id(w.c_z, w.hidden, w.dtype)}:{w.name}"),
                "mfma_busy_frac": counters_for(
                    f"{transition_kernel_id(w.c_z, w.hidden, w.dtype)}:{w.name}").get("mfma_busy_frac"),
                "kernel": dom["kernel"], "avg_launch_ms": dom["ms"],
                "timing": "HIP events around each launch, every launch followed by a whole step",
                "back_to_back_ms": dom.get("back_to_back_ms")}

    result = {
        "metric": METRIC, "value": value, "unit": "pair cells/s per block", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": t_step * 1e3,
        "settle": {"ms": args.settle_ms, "steps": settle_calls,
                   "why": "untimed steps before the warm-up steps, until the clocks settle"},
        "step_ms": spread,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded lengths, N(0,1) singles, "
                                  "N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "B": w.B, "lengths": x.lengths.tolist(), "c_s": w.c_s,
                   "c_z": w.c_z, "hidden": w.hidden, "blocks": w.blocks, "cells": r.cells,
                   "T": r.T, "parallelism": "single GPU",
                   "blocks_via": "nt_pair_chain" if args.chain else "nt_pair_block"},
        "roofline": roofline,
        "kernels": kern,
        "hbm_ceiling": hbm_ceiling(torch),
        "train": train,
        "swiglu_train": swiglu_train,
    }

    if not args.quick:
        result["padded"] = padded_report(x, t_step, packed_peak, r.cells, args, torch, nt)
        result["granularity"] = granularity(x, r, t_step, args, torch, nt)
        del r
        torch.cuda.empty_cache()
        regimes = {}
        for other in pin.WORKLOADS[1:]:
            if other.name == w.name:
                continue
            log(f"regime {other.name}")
            xo = pin.workload_inputs(other.index)
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats()
            base_o = torch.cuda.memory_allocated()
            ro = PackedRunner(xo, torch, nt)
            settle(ro.step, args.settle_ms / 2, torch)  # the GPU idled while inputs were drawn
            to = time_steps(ro.step, args.steps, args.warmup, torch)
            peak_o = torch.cuda.max_memory_allocated() - base_o
            ko = kernel_rooflines(ro, args.kernel_reps)
            regimes[other.name] = {
                "value": ro.cells * other.blocks / to, "ms_per_step": to * 1e3,
                "cells": ro.cells, "blocks": other.blocks,
                "kernels": {k: {"ms": v["ms"], "achieved": v["achieved"], "unit": v["unit"],
                                "frac": v["frac"]} for k, v in ko.items()}}
            if other.blocks > 1:
                regimes[other.name]["granularity"] = granularity(xo, ro, to, args, torch, nt)
            if xo.dtype == "bf16" and other.blocks > 1:
                tro = TrainRunner(xo, torch, nt, ro)
                t_tr = time_steps(tro.step, args.steps, args.warmup, torch)
                regimes[other.name]["train"] = {
                    "value": ro.cells * other.blocks / t_tr, "unit": "pair cells/s per block",
                    "ms_per_step": t_tr * 1e3, "forward_ms": to * 1e3}
                log(f"regime {other.name}: train step {t_tr * 1e3:.3f} ms")
                del tro
            cells_o = ro.cells
            del ro
            torch.cuda.empty_cache()
            if other.blocks > 1:
                regimes[other.name]["padded"] = padded_report(xo, to, peak_o, cells_o, args,
                                                              torch, nt)
            if other.name == "high_variation_x4":
                # the variants on the paper's high-variation regime
                result["rectangular"] = rectangular(xo, args, torch, nt)
                result["non_leading"] = non_leading(xo, args, torch, nt)
        result["regimes"] = regimes
    if not args.no_cpu_baseline and not args.quick:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
