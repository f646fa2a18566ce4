"""CPU oracle for block-sparse video attention: TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct float64 NumPy definitions of every result the
GPU path computes.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product library never does, and shares no
code, table or helper with it.

Modules
  attention  dense masked attention, the symmetric window mask, block-mask
             expansion, block-sparse attention (by definition)
  tiling     T-major tile labels and permutations, cohesion (SICS) by brute
             force over pairs, tiling selection, the sliding-tile block mask
  blocks     min/max block summaries and scores, the budget, top-k with the
             sink and diagonal blocks
  pipeline   the adaptive-tiling recipe end to end

Every function is pinned by the CPU tests in ``tests/test_oracle_*.py``
against closed forms, invariants, library routines and brute force; none is
marked "parity unpinned".

Sources are cited by page title and section:
  [FastVideo windowed_attention.py]  the MLX windowed-attention module page
  [Adaptive tiling (SPADE)]          the mlx-arsenal research note
  [ADR-0001]                         mlx-arsenal "Sparse-attention roadmap for video DiTs"
"""
from . import attention, blocks, pipeline, tiling  # noqa: F401
