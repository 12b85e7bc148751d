"""Plain fp64 CPU oracle of the MapFlow attention-retrieval path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run anything in this directory.  The
product path (the HIP library and its Python binding) never calls it, and this
module imports nothing from that path: the two share no code.

What it computes follows MapFlow ("Accelerating Cross-Model LLM Inference via
Attention Map Reuse", montaan.com/papers/2610.14688, and the PKU-DAIR news
article on it, aitest123.com/news/zaoi86), step by step in the pages' order:

1. block statistics of the sender's causal attention map (article, third
   section, first component: compression first computes block-level
   statistics, then chooses the blocks to keep);
2. block-level Top-p: keep the blocks needed to reach a cumulative attention
   probability p (paper page, highlight 3 "Hardware-Friendly Block-Level Sparse
   Compression");
3. the Block Sparse Row state (paper page, "Practical Implementation Details");
4. retrieval: each reuse receiver head is a linear combination of the sender
   heads with learned weights (paper page, "MapFlow System Design" item 3 and
   highlight 2), multiplied by the receiver's own values and accumulated
   (article, third component; paper page, highlight 4);
5. the same compression computed from the sender's Q and K and the per-row
   log-sum-exp of its scores, without a dense map (article, third section,
   first component);
6. retrieval over a packed batch of sequences (paper page, "Practical
   Implementation Details": the serving integration runs under chunked prefill
   and paged caches), each sequence on its own.

Readings of points the pages leave open (the head-map formula in highlight 2 is
garbled; the statistic, stop rule, tie order, GQA grouping and padding are not
stated) are listed in the repository's design notes and restated at each
function below.

Every function works in float64 on numpy arrays.  Inputs in fp16/bf16/fp32 are
upcast exactly (pass bf16 data as float32 arrays: every bf16 value is an fp32
value).  The loops are deliberately plain: one block, one head at a time.

Parity pins (tests/test_oracle_pins.py) tie every function to something other
than itself: dense causal attention from torch's scaled_dot_product_attention,
brute-force dense decompress-then-matmul, scipy.sparse BSR products, exhaustive
subset search for the Top-p rule, closed-form block-mass identities, a
hand-worked example, and for the Q/K compression torch's causal softmax and
logsumexp, the all-zero-score closed form and plain-loop brute force, and for
the packed batch dense causal attention of each sequence (torch) and a
per-token brute force.  The per-row chain pipeline_row is pinned to the
whole-map path row by row, to the hand-worked example, to torch's attention
(p = 1, identity head map) and to dense brute force, with planted mistakes
(a decision on unrounded masses, transposed tile indices) that must fail.
No function here is "parity unpinned".
"""
from .mapflow_ref import (  # noqa: F401
    n_blocks, block_mass_row, block_mass, topp_row, decision_masses, topp_select,
    bsr_tile, build_bsr, retrieve_row, retrieve, compress, pipeline_row,
    row_lse, QKMap, compress_qk, retrieve_varlen,
)
