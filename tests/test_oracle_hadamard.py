"""Pins for the oracle's Hadamard matrix and block random Hadamard rotation.

The model cards (24B0978 Week 01 Track 2, "How these techniques accelerate
inference on CUDA", paragraph on the random Hadamard transform; 24B0978
Week 02 Track 2, "Recipe") fix that the rotation is a block Hadamard
transform with random signs, that it is orthogonal, that a fast
Walsh-Hadamard butterfly computes it, and that it is undone at restore.
Each test below checks one of those facts, or a closed form that follows
from them, against something other than the oracle's own formula.
"""

import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard as H

ORDERS = [1, 2, 4, 8, 16, 32, 64, 128]


@pytest.mark.parametrize("b", ORDERS)
def test_matches_library_sylvester(b):
    # scipy builds the same Sylvester construction by repeated Kronecker
    # products, a different route from the popcount formula.
    assert np.array_equal(H.hadamard(b), scipy.linalg.hadamard(b))


@pytest.mark.parametrize("b", ORDERS)
def test_rows_orthogonal_exactly(b):
    h = H.hadamard(b)
    assert np.array_equal(h @ h.T, b * np.eye(b, dtype=np.int64))
    assert np.array_equal(h, h.T)
    assert np.all(h[0] == 1) and np.all(h[:, 0] == 1)


def _butterfly(v):
    """Textbook in-place fast Walsh-Hadamard transform (log2(b) add/sub stages)."""
    v = np.array(v, dtype=np.int64)
    b = len(v)
    h = 1
    while h < b:
        for i in range(0, b, 2 * h):
            for j in range(i, i + h):
                a, c = v[j], v[j + h]
                v[j], v[j + h] = a + c, a - c
        h *= 2
    return v


@pytest.mark.parametrize("b", [2, 4, 8, 16, 32, 64, 128])
def test_fast_transform_equals_matrix(b):
    rng = np.random.default_rng(b)
    for _ in range(4):
        x = rng.integers(-1000, 1000, size=b)
        assert np.array_equal(_butterfly(x), H.hadamard(b) @ x)


def test_sign_bit_order():
    k = 128
    bits = np.zeros(4, np.uint32)
    assert np.all(H.signs_from_bits(bits, k) == 1.0)
    bits[0] = 1                     # channel 0
    bits[0] |= np.uint32(1 << 31)   # channel 31
    bits[1] = 1                     # channel 32
    bits[3] = np.uint32(1 << 31)    # channel 127
    d = H.signs_from_bits(bits, k)
    neg = set(np.nonzero(d < 0)[0].tolist())
    assert neg == {0, 31, 32, 127}


def _rand_bits(rng, k):
    return rng.integers(0, 1 << 32, size=k // 32, dtype=np.uint64).astype(np.uint32)


def test_no_signs_is_scaled_hadamard():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 256))
    got = H.rht(x, np.zeros(8, np.uint32))
    h = scipy.linalg.hadamard(128).astype(np.float64)
    want = np.concatenate([x[:, :128] @ h, x[:, 128:] @ h], axis=1) / np.sqrt(128.0)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    # all signs negative flips every output
    got_neg = H.rht(x, np.full(8, 0xFFFFFFFF, np.uint32))
    np.testing.assert_allclose(got_neg, -want, rtol=0, atol=1e-13)


def test_rotation_is_orthonormal():
    rng = np.random.default_rng(2)
    bits = _rand_bits(rng, 128)
    rt = H.rht(np.eye(128), bits)   # row j is R e_j, so this is R^T
    np.testing.assert_allclose(rt @ rt.T, np.eye(128), rtol=0, atol=1e-15 * 128)


def test_one_hot_columns():
    rng = np.random.default_rng(3)
    bits = _rand_bits(rng, 128)
    d = H.signs_from_bits(bits, 128)
    h = scipy.linalg.hadamard(128)
    for j in [0, 1, 5, 63, 64, 127]:
        e = np.zeros(128)
        e[j] = 1.0
        np.testing.assert_allclose(H.rht(e, bits), d[j] * h[:, j] / np.sqrt(128.0), rtol=0, atol=1e-16)


def test_norm_preserved_per_block():
    rng = np.random.default_rng(4)
    k = 1024
    bits = _rand_bits(rng, k)
    x = rng.standard_normal((5, k)) * rng.uniform(0.1, 30, size=(5, 1))
    y = H.rht(x, bits)
    nx = np.linalg.norm(x.reshape(5, -1, 128), axis=2)
    ny = np.linalg.norm(y.reshape(5, -1, 128), axis=2)
    np.testing.assert_allclose(ny, nx, rtol=1e-14)


def test_block_sum_closed_form():
    # Row 0 of H is all ones and every other column of H sums to zero, so the
    # entries of one rotated block sum to sqrt(128) * d0 * x0.  A diagonal
    # applied after H instead of before would break this.
    rng = np.random.default_rng(5)
    k = 512
    bits = _rand_bits(rng, k)
    d = H.signs_from_bits(bits, k)
    x = rng.standard_normal((4, k))
    y = H.rht(x, bits)
    for j in range(k // 128):
        sums = y[:, 128 * j:128 * (j + 1)].sum(axis=1)
        np.testing.assert_allclose(sums, np.sqrt(128.0) * d[128 * j] * x[:, 128 * j], rtol=1e-12, atol=1e-12)


def test_inverse_round_trip():
    rng = np.random.default_rng(6)
    k = 768
    bits = _rand_bits(rng, k)
    x = rng.standard_normal((3, k))
    np.testing.assert_allclose(H.rht_inverse(H.rht(x, bits), bits), x, rtol=0, atol=1e-13)
    np.testing.assert_allclose(H.rht(H.rht_inverse(x, bits), bits), x, rtol=0, atol=1e-13)


def test_blocks_are_independent():
    rng = np.random.default_rng(7)
    k = 512
    bits = _rand_bits(rng, k)
    x = rng.standard_normal(k)
    y0 = H.rht(x, bits)
    x2 = x.copy()
    x2[128:256] += rng.standard_normal(128)
    y1 = H.rht(x2, bits)
    assert np.array_equal(y0[:128], y1[:128]) and np.array_equal(y0[256:], y1[256:])
    assert not np.allclose(y0[128:256], y1[128:256])


def test_fp16_inputs_rotate_exactly_before_scaling():
    # For fp16 inputs the +-1 sums are exact in fp64, so the result times
    # sqrt(128) is the integer combination H (d x), computed here in exact
    # integer arithmetic on the scaled fp16 values.
    rng = np.random.default_rng(8)
    bits = _rand_bits(rng, 128)
    d = H.signs_from_bits(bits, 128).astype(np.int64)
    x16 = rng.standard_normal(128).astype(np.float16)
    xi = (x16.astype(np.float64) * 2.0 ** 24).astype(np.int64)   # exact: fp16 >= 2^-24
    want = scipy.linalg.hadamard(128).astype(np.int64) @ (d * xi)
    got = H.rht(x16, bits) * np.sqrt(128.0) * 2.0 ** 24
    np.testing.assert_allclose(got, want.astype(np.float64), rtol=1e-15, atol=1e-6)
