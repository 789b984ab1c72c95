"""Sylvester Hadamard matrix and the block random Hadamard rotation (oracle).

Test infrastructure only: see the package docstring for who may use it.

[W01] "How these techniques accelerate inference on CUDA", paragraph on the
random Hadamard transform: each weight matrix is rotated by a block Hadamard
transform before quantisation and the inverse rotation is applied on the
other side; the transform is orthogonal; at run time it acts on the
activations while the weight side is folded in offline.  [W02] "Recipe":
the transform is applied per weight block before quantisation and undone at
restore.

Readings taken where the cards are silent:
* ordering: Sylvester (natural) order, ``H[i, j] = (-1)^popcount(i & j)``;
* block: 128, aligned with the quantisation groups;
* the random diagonal ``D`` acts first: ``R = H . D / sqrt(128)`` per block,
  with one sign per input channel; the same ``R`` rotates every weight row
  and every activation row, so ``(R w) . (R x) = w . x``;
* signs arrive as a bit vector: bit ``k & 31`` of word ``k >> 5`` set means
  ``d[k] = -1``.

This module computes the rotation by an explicit matrix-vector product; it
deliberately does not use a fast transform.
"""

from __future__ import annotations

import numpy as np

BLOCK = 128


def hadamard(b: int) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix of order ``b`` (a power of two), int64."""
    if b < 1 or b & (b - 1):
        raise ValueError("order must be a power of two")
    h = np.empty((b, b), dtype=np.int64)
    for i in range(b):
        for j in range(b):
            h[i, j] = -1 if bin(i & j).count("1") % 2 else 1
    return h


def signs_from_bits(bits: np.ndarray, k: int) -> np.ndarray:
    """The ``k`` diagonal entries (+1.0 / -1.0, fp64) encoded by a sign bit vector."""
    bits = np.asarray(bits, dtype=np.uint32)
    if bits.shape != (k // 32,):
        raise ValueError("need k/32 sign words")
    d = np.empty(k, dtype=np.float64)
    for c in range(k):
        bit = (int(bits[c >> 5]) >> (c & 31)) & 1
        d[c] = -1.0 if bit else 1.0
    return d


def rht(x: np.ndarray, sign_bits: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Rotate each length-``block`` slice of every row of ``x`` (fp64 result).

    ``x`` is ``[rows][k]``; block ``j`` of a row becomes
    ``H . (d[j*b:(j+1)*b] * x[:, j*b:(j+1)*b]) / sqrt(b)``.  The product with
    ``H`` is a plain matrix product; the division by ``sqrt(b)`` comes last.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        return rht(x[None, :], sign_bits, block)[0]
    rows, k = x.shape
    if k % block:
        raise ValueError("k must be a multiple of the block")
    d = signs_from_bits(sign_bits, k)
    h = hadamard(block).astype(np.float64)
    out = np.empty_like(x)
    for j in range(k // block):
        sl = slice(j * block, (j + 1) * block)
        out[:, sl] = ((d[sl][None, :] * x[:, sl]) @ h.T) / np.sqrt(float(block))
    return out


def rht_inverse(y: np.ndarray, sign_bits: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Undo ``rht``: ``x = D . H^T . y / sqrt(b)`` per block (fp64)."""
    y = np.asarray(y, dtype=np.float64)
    if y.ndim == 1:
        return rht_inverse(y[None, :], sign_bits, block)[0]
    rows, k = y.shape
    d = signs_from_bits(sign_bits, k)
    h = hadamard(block).astype(np.float64)
    out = np.empty_like(y)
    for j in range(k // block):
        sl = slice(j * block, (j + 1) * block)
        out[:, sl] = d[sl][None, :] * ((y[:, sl] @ h) / np.sqrt(float(block)))
    return out
