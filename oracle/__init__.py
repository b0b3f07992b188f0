"""Reference oracle for the Mamba-2 SSD forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's ``smoke()`` check and the benchmark's CPU-baseline
leg may import this package. The GPU product path (``state_space_sequence_chunk_amd``)
never imports, links or calls anything here, and nothing here imports the product.

Contents
--------
``forward``            fp64 token-by-token recurrence (C, ``ssd_oracle.c``), the plain
                       definition of the forward pass (page "Accelerating Mamba-2 with
                       High-Performance Forward Pass Kernels in NVIDIA CUDA Tile",
                       section "Mamba-2 architecture", the core recurrence).
``forward_pairs``      the same recurrence on a chosen subset of (batch, head) pairs of a
                       full-size problem, for sampled parity at sizes where the whole
                       oracle would be too slow.
``chunk_cumsum_log2``  the per-chunk cumulative decay in base-2 log space (same page,
                       section "Kernel 1: Computing cumulative sums"): the inclusive sum
                       of A*dt from the chunk's first token, times log2(e).
``forward64``          the recurrence with float64 inputs (``ssd_oracle_grad.c``), used
                       by the finite-difference checks of the gradients.
``backward``           fp64 reverse-mode gradients of the recurrence with respect to x,
                       dt, A, B, C, D and h0 (``ssd_oracle_grad.c``).

Everything computes in float64 from float32-representable inputs (bf16 and fp32 input
values are exact in float32).
"""
from .ssd_oracle import (  # noqa: F401
    backward,
    build,
    chunk_cumsum_log2,
    forward,
    forward64,
    forward_pairs,
    library_path,
)
