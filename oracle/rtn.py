"""Weight-side rotation and round-to-nearest group quantisation (oracle).

Test infrastructure only: see the package docstring for who may use it.

[W01] paragraph on group-wise affine integer quantisation: the weight is
kept as integer codes with one fp16 scale and one fp16 zero point per group
of 128 consecutive entries along the reduction dimension, and a weight is
recovered as ``w = (q - z) * s``.  [W02] "Recipe" / "Recipe (exact)": the
embedding is quantised by round-to-nearest (RTN) at 8 bits, group 128; the
other stage uses 6 bits, group 128.  [W01] paragraph on the Hadamard
transform: the weight is rotated before it is quantised.

Readings taken where the cards are silent (the cards name RTN but give no
formula):
* asymmetric min-max with the range stretched to contain 0:
  ``lo = min(min(v), 0)``, ``hi = max(max(v), 0)``;
* the scale is rounded to fp16 (nearest, ties to even) *before* the zero
  point and the codes are computed from it: ``s = fp16((hi - lo) / qmax)``,
  and ``s = 1`` if that rounds to 0 (an all-zero group);
* ``z = clamp(rint(-lo / s), 0, qmax)`` (an integer, exact in fp16);
* ``q = clamp(rint(v / s + z), 0, qmax)``;
* all of it in fp64 on the fp32 rotated weight; ``rint`` rounds half to even.
The rotated weight is rounded to fp32 once, after the fp64 rotation.
"""

from __future__ import annotations

import numpy as np

from .hadamard import rht, BLOCK

GROUP = 128


def rotate_weight(w: np.ndarray, sign_bits: np.ndarray, keep_fp64: bool = False) -> np.ndarray:
    """``W' = R W`` row by row: every weight row gets the activations' rotation.

    Returns the fp32 rounding of the fp64 result (``keep_fp64`` returns the
    fp64 value itself, used to check that the rotation preserves the layer).
    """
    wp = rht(np.asarray(w, dtype=np.float64), sign_bits, BLOCK)
    return wp if keep_fp64 else wp.astype(np.float32)


def rtn(w: np.ndarray, bits, group: int = GROUP):
    """Round-to-nearest asymmetric quantisation per (row, group of ``group`` along K).

    ``w`` is fp32 ``[n][k]``.  ``bits`` is an int (3, 4, 6 or 8) or an array
    with one width per row.  Returns ``(q, s, z)``: ``q`` uint8 ``[n][k]``,
    ``s`` and ``z`` float16 ``[n][k/group]``.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % group:
        raise ValueError("k must be a multiple of the group")
    g = k // group
    rowbits = np.broadcast_to(np.asarray(bits, dtype=np.int64), (n,))
    qmax = ((1 << rowbits) - 1).astype(np.float64)[:, None]            # [n][1]

    v = w.astype(np.float64).reshape(n, g, group)
    lo = np.minimum(v.min(axis=2), 0.0)                                 # [n][g]
    hi = np.maximum(v.max(axis=2), 0.0)
    s16 = ((hi - lo) / qmax).astype(np.float16)
    s16[s16 == 0] = np.float16(1.0)
    s = s16.astype(np.float64)
    z = np.clip(np.rint(-lo / s), 0.0, qmax)
    q = np.clip(np.rint(v / s[:, :, None] + z[:, :, None]), 0.0, qmax[:, :, None])
    return q.reshape(n, k).astype(np.uint8), s16, z.astype(np.float16)


def prepare(w: np.ndarray, sign_bits, bits):
    """Offline weight preparation: rotate (if ``sign_bits`` is given), then RTN."""
    wp = rotate_weight(w, sign_bits) if sign_bits is not None else np.asarray(w, np.float32)
    return rtn(wp, bits)
