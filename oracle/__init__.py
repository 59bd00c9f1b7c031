"""CPU oracle for the GNN-layer hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import, call, link or execute anything in this package.  The product path (the
HIP library and its Python binding) never touches it and shares no code with
it: no kernels, headers, helpers or tables.

What it computes, in float64 unless noted, and where each step is defined:

* ``csr.build``  -- the normalised adjacency of one partition.  The modified
  adjacency D^-1/2 (A+I) D^-1/2 with D the degrees of A+I ("Reducing
  Communication in Graph Neural Network Training", background section on GNN
  forward propagation; Sylvie, "Forward Propagation" paragraph), the
  GraphSAGE mean, the HALO node set of a partition (Sylvie, "Graph Engine";
  DIGEST, "pull" operation in the system-design section) and the transposed
  matrix that the backward pass multiplies by (CAGNET page: A and A^T are
  kept distinct).
* ``layers``     -- the GCN layer sigma(A^T H W + b) of the CAGNET page's
  forward-propagation equation with the DIGEST split P_in H_in + P_out H~_out
  (DIGEST, matrix form of the modified forward pass), the GraphSAGE-mean layer
  sigma([h_v | mean_u h_u] W + b) (Sylvie, aggregation then update with the
  node's own vector), and their backward passes (CAGNET: backpropagation uses
  the same SpMM and GEMM primitives).
* ``native``     -- the fp64 CSR SpMM in plain C (each output row summed over
  its entries in ascending order).
* ``lowbit``     -- Sylvie's Low-bit Module (b-bit stochastic quantization of
  halo rows with a per-row scale and zero-point; dequantization) with the
  Philox4x32-10 counter-based generator for its draws, and DIGEST's push of
  a partition's rows into the representation store (plus the accumulating
  form used for halo gradients).
* ``gat``        -- the graph-attention layer the pages name (GAT, Velickovic
  et al. 2018; Sylvie, first section; DIGEST, evaluation section), in its
  textbook form since the pages print no formulas: per-entry LeakyReLU
  scores, a softmax over each row, the attention-weighted sum of the
  transformed rows, heads concatenated, and its backward pass.

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that takes it.  Every function is pinned by tests
under ``tests/`` that do not re-type its formulas: closed forms, invariants,
brute force on tiny inputs and finite differences.
"""
from . import csr, gat, layers, lowbit, native  # noqa: F401
