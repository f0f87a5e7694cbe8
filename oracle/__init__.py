"""Test infrastructure: the plain CPU oracle for scaled dot-product attention.

This package is NOT part of the product path.  Only the tests, the smoke check
and the CPU-baseline leg of the benchmark may import it; the HIP library never
does, and the two share no code.

What it computes (fp64, the textbook definition, no tiling, no online softmax):

    S = scale * Q K^T                       per (batch, query head)
    S[i, j] = -inf where key j is not allowed for query i
    P = row-wise softmax(S)
    O = P V,   lse_i = log sum_j exp(S[i, j])

and, in `sdpa_bwd`, the exact gradients dQ, dK, dV of that function given
dO, written out by the chain rule (dV = P^T dO, dP = dO V^T, the softmax
Jacobian for dS, dQ = scale dS K, dK = scale dS^T Q).

Sources (page titles as printed on the pages; see each function for the exact
passage):
  * "SpAtten: Efficient Sparse Attention Architecture with Cascade Token and
    Head Pruning, HPCA 2021" (review page), Background - Attention Mechanism:
    the score Q K^T / sqrt(D) and Softmax(score) V; Algorithm Optimization -
    D. Progressive Quantization: the probability p_i = exp(s_i)/sum_j exp(s_j).
  * The self-attention explainer page (palettepath-it, "셀프 어텐션 메커니즘의
    본질적 가치와 미래 동력"), sections on scaled dot-product scoring, softmax
    normalisation and weighted sum, multi-head attention, padding masking and
    look-ahead masking.
  * The O(n^2) tutorial page (devhandbook), "Local Window Attention" strategy
    and Example 7 (variable-length padding masks).
  * "Attentions Under the Microscope" summary page, Methodology: grouped-query
    attention and sliding-window attention named as benchmarked variants.

Readings of points the pages leave open are listed in the docstring of
`allowed_mask`.

Pinning: every function here is checked in tests/test_oracle_pins.py against
brute force (`oracle.brute`), closed forms, published invariants and an
independent library routine.  No function here is "parity unpinned".
"""

from .sdpa import (  # noqa: F401
    allowed_mask,
    attention,
    attention_rows,
    probabilities,
    row_positions,
)
from .sdpa_bwd import attention_backward  # noqa: F401
from . import brute  # noqa: F401
from . import fp8  # noqa: F401
