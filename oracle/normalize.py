"""Per-vector L2 normalisation of q and k (fp64), the optional pre-step of the
token-by-token forward (FLA DeltaNet article, section 5: the in-kernel L2
normalisation option of q and k).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Reading of the pages: they name the option but not its formula. The plainest
form, used here and by the GPU kernel, divides each head's vector by
sqrt(sum of squares + eps) with eps = 1e-6, so that a zero vector stays zero
instead of producing a division by zero.
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6


def l2_normalize(x: np.ndarray, eps: float = L2_EPS) -> np.ndarray:
    """x / sqrt(sum(x**2, last axis) + eps), in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
