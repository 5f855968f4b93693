"""Output-relative (POEM-style) block-sparse causal attention prefill for MI355X.

The hot path lives in libpoem.so (hand-written HIP for gfx950 behind a C ABI,
declared in include/poem.h). This package holds the ctypes binding
(``_lib``), the in-tree build (``build``) and the seeded synthetic inputs
(``synth``).
"""
from ._lib import (POEM_BF16, POEM_FP32, PoemError, Problem, SelectWorkspace, SparseWorkspace,  # noqa: F401
                   csr_capacity, dense_prefill, flops_dense, load, max_visible_blocks, num_tiles, select,
                   select_workspace_bytes, sparse_prefill, sparse_workspace_bytes, version)
