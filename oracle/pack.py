"""Bit placement of integer codes into 32-bit words (oracle).

Test infrastructure only: see the package docstring for who may use it.

[W01] paragraph on the absence of unstructured sparsity: every tensor stays
a dense packed integer array with a regular stride.  [GPTQ3] "CUDA speedup
potential": packed int3 codes are read directly by the kernel.  [MIX]
"Method, selection, and reproduction": the stream holds dense mixed-width
codes in 64-row blocks with a byte selector per block.

Layout (the cards fix none of it; this is the reading used throughout):
* codes of one output row are contiguous along K; rows follow each other;
  a row of ``k`` codes at ``b`` bits occupies ``k*b/32`` words;
* int4: 8 codes per word, code ``j`` of the word in bits ``[4j, 4j+4)``
  (lowest nibble first); int8: 4 codes per word, byte 0 lowest;
* int3: 32 codes per 3 words, int6: 16 codes per 3 words; the three words
  form one 96-bit little-endian integer ``w0 | w1 << 32 | w2 << 64`` and
  code ``j`` of the run occupies bits ``[b*j, b*j + b)`` of it, so some
  codes straddle two words;
* mixed width: output rows are cut into 64-row blocks; block ``i`` is coded
  at ``sel[i]`` bits (6 or 8) with the uniform layout above; blocks are
  concatenated with no padding, and block ``i`` starts at word
  ``off[i] = sum over earlier blocks of 64 * k * sel / 32``.

Packing here is scalar: every code is placed bit by bit with Python
integers, so the layout can be read straight off the code.
"""

from __future__ import annotations

import numpy as np

RUN = {3: (32, 3), 4: (8, 1), 6: (16, 3), 8: (4, 1)}   # bits -> (codes per run, words per run)
MIXED_ROWS = 64


def words_per_row(bits: int, k: int) -> int:
    codes, words = RUN[bits]
    if k % codes:
        raise ValueError(f"k={k} is not a multiple of {codes} for {bits}-bit codes")
    return k // codes * words


def pack_row(codes_row, bits: int) -> np.ndarray:
    """Pack one row of codes (each < 2**bits) into uint32 words."""
    per_run, wpr = RUN[bits]
    codes_row = [int(c) for c in codes_row]
    out = []
    for r0 in range(0, len(codes_row), per_run):
        acc = 0
        for j, c in enumerate(codes_row[r0:r0 + per_run]):
            if not 0 <= c < (1 << bits):
                raise ValueError("code out of range")
            acc |= c << (bits * j)
        for w in range(wpr):
            out.append((acc >> (32 * w)) & 0xFFFFFFFF)
    return np.array(out, dtype=np.uint32)


def unpack_row(words_row, bits: int, k: int) -> np.ndarray:
    """Inverse of ``pack_row``: ``k`` codes from one row of words."""
    per_run, wpr = RUN[bits]
    words_row = [int(w) for w in words_row]
    out = []
    for r in range(k // per_run):
        acc = 0
        for w in range(wpr):
            acc |= words_row[r * wpr + w] << (32 * w)
        for j in range(per_run):
            out.append((acc >> (bits * j)) & ((1 << bits) - 1))
    return np.array(out, dtype=np.uint8)


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """Uniform width: uint8 ``[n][k]`` codes -> uint32 ``[n][k*bits/32]``."""
    q = np.asarray(q)
    n, k = q.shape
    out = np.empty((n, words_per_row(bits, k)), dtype=np.uint32)
    for i in range(n):
        out[i] = pack_row(q[i], bits)
    return out


def unpack(words: np.ndarray, bits: int, n: int, k: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint32).reshape(n, words_per_row(bits, k))
    out = np.empty((n, k), dtype=np.uint8)
    for i in range(n):
        out[i] = unpack_row(words[i], bits, k)
    return out


def block_offsets(sel: np.ndarray, k: int) -> np.ndarray:
    """Word offset of every 64-row block, plus the total, as uint64 ``[blocks+1]``."""
    off = [0]
    for b in np.asarray(sel):
        off.append(off[-1] + MIXED_ROWS * words_per_row(int(b), k))
    return np.array(off, dtype=np.uint64)


def pack_mixed(q: np.ndarray, sel: np.ndarray):
    """Mixed width: returns (flat uint32 words, uint64 block offsets)."""
    q = np.asarray(q)
    n, k = q.shape
    if n % MIXED_ROWS or len(sel) != n // MIXED_ROWS:
        raise ValueError("need one selector per 64 rows")
    off = block_offsets(sel, k)
    out = np.empty(int(off[-1]), dtype=np.uint32)
    for i, b in enumerate(np.asarray(sel)):
        b = int(b)
        if b not in (6, 8):
            raise ValueError("mixed-width selectors must be 6 or 8")
        wpr = words_per_row(b, k)
        for r in range(MIXED_ROWS):
            row = i * MIXED_ROWS + r
            start = int(off[i]) + r * wpr
            out[start:start + wpr] = pack_row(q[row], b)
    return out, off


def unpack_mixed(words: np.ndarray, sel: np.ndarray, n: int, k: int) -> np.ndarray:
    off = block_offsets(sel, k)
    out = np.empty((n, k), dtype=np.uint8)
    for i, b in enumerate(np.asarray(sel)):
        b = int(b)
        wpr = words_per_row(b, k)
        for r in range(MIXED_ROWS):
            start = int(off[i]) + r * wpr
            out[i * MIXED_ROWS + r] = unpack_row(words[start:start + wpr], b, k)
    return out
