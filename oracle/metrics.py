"""Action-space error metrics of the paper's §III-E, Eq. 5 -- test infrastructure only.

e_inf is the largest absolute entry-wise difference; e_rel is the Euclidean norm
of the flattened difference over the Euclidean norm of the flattened reference.
When the reference norm is zero the relative error is undefined and the
absolute norm of the difference is reported instead.
"""
from __future__ import annotations

import numpy as np


def e_inf(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - ref)))


def e_rel(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    diff = float(np.linalg.norm(a - ref))
    den = float(np.linalg.norm(ref))
    return diff if den == 0.0 else diff / den
