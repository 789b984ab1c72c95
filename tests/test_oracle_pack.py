"""Pins for the oracle's code packing (uniform and mixed width).

The cards fix a dense packed code array with a regular stride
(24B0978 Week 01 Track 2, "How these techniques accelerate inference on
CUDA", paragraph on sparsity), packed int3 read directly by the kernel
(24B0908 card, "CUDA speedup potential") and dense mixed 6/8-bit codes in
64-row blocks with byte selectors (25M2111 card, "Method, selection, and
reproduction").  The bit placement itself is this project's reading; the
worked examples in ``golden/pack_examples.json`` were derived by hand from
it and pin the packer.
"""

import json
import os

import numpy as np
import pytest

from oracle import pack as P

GOLD = os.path.join(os.path.dirname(__file__), "golden", "pack_examples.json")


def test_worked_examples():
    for c in json.load(open(GOLD))["cases"]:
        want = [int(w, 16) for w in c["words"]]
        got = P.pack_row(c["codes"], c["bits"]).tolist()
        assert got == want, c["why"]
        assert P.unpack_row(want, c["bits"], len(c["codes"])).tolist() == c["codes"], c["why"]


@pytest.mark.parametrize("bits,k,words", [(3, 128, 12), (4, 128, 16), (6, 128, 24), (8, 128, 32),
                                          (4, 2560, 320), (3, 9728, 912), (6, 4096, 768)])
def test_words_per_row(bits, k, words):
    assert P.words_per_row(bits, k) == words


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
def test_every_value_at_every_position(bits):
    per_run = {3: 32, 4: 8, 6: 16, 8: 4}[bits]
    for j in range(per_run):
        for v in range(1 << bits):
            codes = [0] * per_run
            codes[j] = v
            words = P.pack_row(codes, bits)
            assert P.unpack_row(words, bits, per_run).tolist() == codes
            # exactly popcount(v) bits set, nothing leaks elsewhere
            assert sum(bin(int(w)).count("1") for w in words) == bin(v).count("1")


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
def test_round_trip_matrix(bits):
    rng = np.random.default_rng(bits)
    q = rng.integers(0, 1 << bits, size=(5, 256), dtype=np.uint8)
    w = P.pack(q, bits)
    assert w.shape == (5, P.words_per_row(bits, 256))
    assert np.array_equal(P.unpack(w, bits, 5, 256), q)


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
def test_rows_are_contiguous_runs(bits):
    # row r of the packed matrix depends only on row r of the codes, and
    # packing a concatenation of runs concatenates their words
    rng = np.random.default_rng(40 + bits)
    q = rng.integers(0, 1 << bits, size=(3, 256), dtype=np.uint8)
    w = P.pack(q, bits)
    half = P.words_per_row(bits, 128)
    for r in range(3):
        assert np.array_equal(w[r], P.pack_row(q[r], bits))
        assert np.array_equal(w[r, :half], P.pack_row(q[r, :128], bits))
        assert np.array_equal(w[r, half:], P.pack_row(q[r, 128:], bits))


def test_block_offsets_hand_values():
    # 64 rows x 128 codes: 6-bit block = 64*24 = 1536 words, 8-bit = 64*32 = 2048
    off = P.block_offsets(np.array([6, 8, 6], np.uint8), 128)
    assert off.tolist() == [0, 1536, 3584, 5120]


@pytest.mark.parametrize("width", [6, 8])
def test_uniform_selector_equals_uniform_width(width):
    rng = np.random.default_rng(width)
    q = rng.integers(0, 1 << width, size=(192, 128), dtype=np.uint8)
    sel = np.full(3, width, np.uint8)
    words, off = P.pack_mixed(q, sel)
    assert np.array_equal(words, P.pack(q, width).ravel())
    assert off[-1] == words.size


def test_mixed_round_trip_and_block_content():
    rng = np.random.default_rng(50)
    sel = np.array([6, 8, 8, 6], np.uint8)
    q = np.empty((256, 256), np.uint8)
    for i, b in enumerate(sel):
        q[64 * i:64 * (i + 1)] = rng.integers(0, 1 << int(b), size=(64, 256))
    words, off = P.pack_mixed(q, sel)
    assert np.array_equal(P.unpack_mixed(words, sel, 256, 256), q)
    for i, b in enumerate(sel):
        blk = words[int(off[i]):int(off[i + 1])]
        assert np.array_equal(blk, P.pack(q[64 * i:64 * (i + 1)], int(b)).ravel())


def test_rejects_bad_codes():
    with pytest.raises(ValueError):
        P.pack_row([16] + [0] * 7, 4)
    with pytest.raises(ValueError):
        P.pack_mixed(np.zeros((64, 128), np.uint8), np.array([4], np.uint8))
