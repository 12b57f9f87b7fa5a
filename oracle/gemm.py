"""fp64 CPU oracle for the linear-layer GEMM ``C = A W^T``.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package. It shares
no code with the HIP library and imports nothing from it.

What it follows. The write-ups of "Defeating Nondeterminism in LLM Inference" make the matrix
multiplication batch invariant by a fixed tiling without Split-K (xitu-tech.com report, section
构建确定性解决方案, matrix multiplication item; neican.ai insight page, section
技术原理与创新点解析, matmul item). Tiling changes only rounding, so the oracle is the product
itself, ``C[i][j] = sum_k A[i][k] W[j][k]``, in float64 on the exact input values.

Pins (tests/test_oracle_gemm.py): pure-Python loops on tiny matrices, identity and one-hot
closed forms, and linearity in A.
"""

from __future__ import annotations

import numpy as np


def gemm(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """``a [M][K]`` times the transpose of ``w [N][K]``, float64 ``[M][N]``."""
    return np.asarray(a, np.float64) @ np.asarray(w, np.float64).T
