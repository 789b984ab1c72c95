"""Tied-embedding gather (oracle).

Test infrastructure only: see the package docstring for who may use it.

[W02] "Recipe": the token embedding is tied to the output head and stored as
round-to-nearest codes (8 bits, group 128), so one table of codes, scales and
zero points gives both the head's weights and the embedding rows.  Row ``i``
of a gather is table row ``ids[i]`` dequantised ([W01] paragraph on
group-wise affine integer quantisation: ``w = (q - z) * s`` per group of 128
along the row), computed in fp64 and rounded once to the output type.

The cards do not say what an invalid token id gives; the library's reading
is a row of zeros, and so is this one's.
"""

from __future__ import annotations

import numpy as np

from .linear import dequant


def embed(q, s, z, ids, out_dtype=np.float16) -> np.ndarray:
    """``out[i] = (q[ids[i]] - z[ids[i]]) * s[ids[i]]`` (per group), rounded once to ``out_dtype``."""
    q = np.asarray(q)
    n, k = q.shape
    ids = np.asarray(ids, dtype=np.int64).ravel()
    out = np.zeros((len(ids), k), dtype=np.float64)
    for i, r in enumerate(ids):
        if 0 <= r < n:
            out[i] = dequant(q[r:r + 1], np.asarray(s)[r:r + 1], np.asarray(z)[r:r + 1])[0]
    return out.astype(out_dtype)
