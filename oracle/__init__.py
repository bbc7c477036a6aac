"""Float64 CPU oracle for the SALA hybrid attention layer group.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP kernels are checked against.  Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``hybrid_sparse_linear_amd``) never imports,
links or calls anything here, and nothing here imports the product path.

Every function works in float64 on NumPy arrays.  Callers widen the exact
bf16 / fp32 values that the GPU receives to float64 before calling in.

Sources (the pages describing the method):
  [P1] "MiniCPM-SALA: Hybridizing Sparse and Linear Attention for Efficient
       Long-Context Modeling", abstract (fugumt.com summary of arXiv 2602.11761).
  [P2] same title, gist.science (Japanese), technical summary (技術概要),
       sections 1 (problem), 2.1 (hybrid attention), 2.2 (HyPE), 4.3 (speed).
  [P3] same title, gist.science (German), technical summary
       ("Technische Zusammenfassung"), section 2 "Methodik",
       subsection "Architektur-Hybridisierung".
  [P4] "Punctuation-aware Hybrid Trainable Sparse Attention for Large
       Language Models", abstract (fugumt.com, arXiv 2601.02819).
  [P5] related-paper entry "FlashAttention: Fast and Memory-Efficient Exact
       Attention with IO-Awareness" on the fugumt.com page for arXiv 2607.21752.

Modules:
  linear  -- Lightning (causal, decayed) linear attention: quadratic
             definition, chunked form, recurrent form, one decode step.
  sparse  -- block pooling, block scoring, top-k block selection with forced
             initial/local blocks, and softmax attention restricted to the
             selected token set (prefill and decode).
  neighbours -- the linear layer's QK RMS normalisation, HyPE RoPE and output
             gate, and the layer composed with them (prefill and decode).
  backward -- gradients of the linear layer (dq, dk, dv, d state_in) and of
             the sparse attention at a fixed selection (dq, dk, dv), for the
             continual training the pages describe.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_linear.py``, ``tests/test_oracle_sparse.py``,
``tests/test_oracle_neighbours.py`` and ``tests/test_oracle_backward.py``
(central finite differences, an independent chunked form, torch autograd of
scaled_dot_product_attention in float64) against
exact rational brute force, closed forms, special cases that reduce to a
library routine, or invariants.  The *choice* of the method's unstated
details (no feature map or normaliser in linear attention, the decay form,
mean pooling, the forced-block rule) is a reading of the pages; those
readings are listed in the design notes and are pinned only by the
internal invariants, not by any number on the pages.
"""

from . import backward, linear, neighbours, sparse  # noqa: F401
