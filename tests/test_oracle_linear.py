"""Pins for the oracle's dequantisation and contraction.

The cards fix w = (q - z) * s with s and z shared by the 128 consecutive
weights of a group along the reduction dimension, the scale applied once to
a group's partial sum (24B0978 Week 01 Track 2, "How these techniques
accelerate inference on CUDA", paragraph on group-wise quantisation), and
activations rotated with the rotation folded into the weights (same card,
paragraph on the random Hadamard transform).  The tests pin the contraction
against a library product and exact integer arithmetic, the group mapping
against hand values, and the whole pipeline against the unquantised layer.
"""

import numpy as np
import pytest

from oracle import hadamard as H
from oracle import linear as L
from oracle import rtn as R


def test_triple_loop_matches_library_product():
    rng = np.random.default_rng(0)
    for (m, n, k) in [(1, 7, 128), (3, 33, 256), (16, 5, 1024)]:
        w = rng.standard_normal((n, k))
        x = rng.standard_normal((m, k))
        got = L.contract(w, x)
        want = x @ w.T
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_triple_loop_independent_of_threads():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((97, 384))
    x = rng.standard_normal((2, 384))
    assert np.array_equal(L.contract(w, x, threads=1), L.contract(w, x, threads=5))


def test_integer_special_case_is_exact():
    # 8-bit codes with s = 1 and z = 0 and integer activations: the layer is
    # an exact integer matrix product.
    rng = np.random.default_rng(2)
    n, k = 40, 384
    q = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    s = np.ones((n, k // 128), np.float16)
    z = np.zeros((n, k // 128), np.float16)
    x = rng.integers(-50, 50, size=(3, k))
    got = L.linear(q, s, z, x.astype(np.float16))
    want = x.astype(np.int64) @ q.astype(np.int64).T
    assert np.array_equal(got, want.astype(np.float64))


def test_group_index_hand_values():
    # two groups along K: codes 3, s = (0.5, 2), z = (1, 2) -> weights 1 then 2
    q = np.full((1, 256), 3, np.uint8)
    s = np.array([[0.5, 2.0]], np.float16)
    z = np.array([[1.0, 2.0]], np.float16)
    w = L.dequant(q, s, z)
    assert np.all(w[0, :128] == 1.0) and np.all(w[0, 128:] == 2.0)
    x = np.concatenate([np.ones(128), np.zeros(128)]).astype(np.float16)
    assert L.linear(q, s, z, x)[0, 0] == 128.0
    x = np.concatenate([np.zeros(128), np.ones(128)]).astype(np.float16)
    assert L.linear(q, s, z, x)[0, 0] == 256.0


def test_non_integer_zero_point_hand_value():
    q = np.array([[0, 1, 2, 3] * 32], np.uint8)
    s = np.array([[0.25]], np.float16)
    z = np.array([[1.5]], np.float16)
    w = L.dequant(q, s, z)
    assert w[0, :4].tolist() == [-0.375, -0.125, 0.125, 0.375]


def test_accumulator_form_identity():
    # sum_k (q - z) s x = sum_g s_g (sum_{k in g} q x - z_g sum_{k in g} x)
    rng = np.random.default_rng(3)
    n, k, m = 20, 512, 4
    q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    s = rng.uniform(0.01, 0.2, size=(n, k // 128)).astype(np.float16)
    z = rng.uniform(0, 15, size=(n, k // 128)).astype(np.float16)
    x = rng.standard_normal((m, k)).astype(np.float16)
    got = L.linear(q, s, z, x)
    xg = x.astype(np.float64).reshape(m, k // 128, 128)
    qg = q.astype(np.float64).reshape(n, k // 128, 128)
    qx = np.einsum("ngc,mgc->mng", qg, xg)
    xs = xg.sum(axis=2)                                   # [m][g]
    want = (s.astype(np.float64)[None] * (qx - z.astype(np.float64)[None] * xs[:, None, :])).sum(axis=2)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_rotated_quantised_layer_tracks_the_float_layer():
    # End to end: rotate + quantise the weight, rotate the activations, and
    # the result stays within the summed rounding error of the weights.
    rng = np.random.default_rng(4)
    n, k = 48, 1024
    bits = rng.integers(0, 1 << 32, size=k // 32, dtype=np.uint64).astype(np.uint32)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((2, k)).astype(np.float16)
    q, s, z = R.prepare(w, bits, 8)
    y = L.linear(q, s, z, x, bits)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    xr = np.abs(H.rht(x.astype(np.float64), bits))
    g = np.arange(k) // 128
    half_step = s.astype(np.float64)[:, g] / 2                     # [n][k]
    wp = R.rotate_weight(w, bits).astype(np.float64)
    bound = xr @ (half_step + np.abs(wp) * 2.0 ** -24).T + 1e-12
    assert np.all(np.abs(y - exact) <= bound)
    # and the error is far below the bound on average (errors cancel)
    assert np.linalg.norm(y - exact) < 0.2 * np.linalg.norm(bound)


def test_head_without_rotation_is_plain_dequant_product():
    rng = np.random.default_rng(5)
    n, k = 30, 256
    q = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, size=(n, 2)).astype(np.float16)
    z = rng.integers(0, 256, size=(n, 2)).astype(np.float16)
    x = rng.standard_normal((1, k)).astype(np.float16)
    w = (q.astype(np.float64) - np.repeat(z.astype(np.float64), 128, axis=1)) * np.repeat(s.astype(np.float64), 128, axis=1)
    np.testing.assert_allclose(L.linear(q, s, z, x), x.astype(np.float64) @ w.T, rtol=1e-13, atol=1e-13)
