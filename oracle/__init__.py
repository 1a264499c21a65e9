"""CPU oracle for the packed single-pair-single block. TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package. The GPU library
never routes through it, and it shares no code with the GPU path: the only
module both sides use is ``pair_inputs`` (seeded draws, no block arithmetic).

Everything is float64 numpy, computed from the exact values of the stored
(fp32 or bf16) inputs with no intermediate rounding. Source: the DanLing
NestedTensor paper (arXiv 2609.30379):

* Section 3, Equation 1 - the block: pair cells are the sum of a row
  projection and a column projection of the singles, a residual feature
  transition updates every cell, and the mean over the column axis, projected
  back to single width, is added to the singles. The block returns both.
* Section 3.1, Equation 2 - packed storage: a sample's ragged prefix is
  collapsed and samples are concatenated; offsets accumulate the packed row
  counts (N_i for singles, N_i^2 for square pairs).
* Section 3.2, Equation 3 - the packed row of ragged coordinates (a, b) of
  sample i is o_i + a * N_i + b for a square pair.
* Section 3.2, Equation 4 - the column sum groups cells of one sample and
  row; the square mean also divides by N_i.
* Figure 2 - for lengths (2, 3) five singles become thirteen cells and the
  sample offsets go from [0, 2, 5] to [0, 4, 13].
* Figure 3 - the row operand is the left projection (unsqueeze(-2)), the
  column operand the right projection (unsqueeze(-3)); the mean is taken over
  dim=-2 of the logical pair shape, i.e. over columns.
* Appendix A - structural invariants (o_0 = 0, o_{i+1} - o_i = p_i,
  o_B = total; zero-volume elements have coincident offsets) and the
  reference-semantics contract: a sample-local packed result, read logically,
  equals the dense per-sample computation.

backward.py holds the gradients: Equation 5's sample-weighted squared loss
(Appendix A.1) over the returned singles and pair state, and the chain rule
through every step of the block, in reverse.

The block's transition is z + relu(z W1^T) W2^T (a two-layer ReLU MLP without
normalisation, the transition of the measured workloads). The paper's own
pre-normalised SwiGLU transition (Eq. 1 with h o LN; Appendix A.1, expansion
four) is here too, as transition_swiglu: LN over the c_z features with affine
gamma, beta and eps = 1e-5 (PyTorch's LayerNorm defaults), then
(silu(x Wg^T) * (x Wu^T)) Wd^T without biases - the plainest reading, as the
pages give SwiGLU's structure but not its formula. Weights are stored
[out, in] as in the paper's V' = V W^T + b (Section 3.3), without biases.

Pins (tests/test_oracle_pins.py) tie every function here to something
outside itself: the Figure 2 worked example, a hand-computed block, closed
forms, brute-force scalar loops, the padded-then-masked and gather forms, and
sample-permutation / batch-splitting invariance. No function is left
unpinned.
"""
from .pair_block import (  # noqa: F401
    partition, decode_cells, broadcast, transition, reduce_mean, project,
    block, chain, block_padded_masked, block_gather, block_bruteforce,
    round_bf16, bf16_bits, block_cells, block_rows, dense_block, broadcast_cells,
    layer_norm, transition_swiglu, block_swiglu, chain_swiglu,
    partition_rect, decode_cells_rect, broadcast_rect, reduce_mean_rect, block_rect,
)
from .backward import (  # noqa: F401
    loss_weights, loss_eq5, reduce_mean_backward, broadcast_backward, transition_backward,
    block_backward, chain_loss, chain_backward, block_nl, block_backward_nl,
    layer_norm_backward, transition_swiglu_backward, block_swiglu_backward, chain_swiglu_loss,
    chain_swiglu_backward,
)
