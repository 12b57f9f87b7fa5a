"""fp64 CPU oracle for RMSNorm.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package. It shares
no code with the HIP library and imports nothing from it.

What it follows. The write-ups of "Defeating Nondeterminism in LLM Inference" list RMSNorm
among the three operators made batch invariant, by reducing each row with one data-parallel
strategy at every batch size (xitu-tech.com report, section 构建确定性解决方案, RMSNorm item;
neican.ai insight page, section 技术原理与创新点解析, RMSNorm item). They give no formula; the
oracle takes the usual definition, ``y = x / sqrt(mean(x^2) + eps) * w`` over the hidden
dimension of each row, in float64 on the exact input values the GPU receives.

Pins (tests/test_oracle_rmsnorm.py): torch's own ``rms_norm`` in float64, a pure-Python loop on
tiny rows, closed forms (constant rows), scale invariance at eps = 0, and the mean square of
``y / w`` equal to ``ms / (ms + eps)``.
"""

from __future__ import annotations

import numpy as np


def rmsnorm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise RMSNorm of ``x [rows][hidden]`` with ``weight [hidden]``, float64."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(weight, np.float64)[None, :]
