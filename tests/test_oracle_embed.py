"""Pins for the oracle's tied-embedding gather.

The table of the output head is also the token embedding (24B0978 Week 02
Track 2, "Recipe": embed_tokens tied to lm_head, RTN 8-bit, group 128), so a
gathered row is the dequantised table row, w = (q - z) * s per group of 128
(24B0978 Week 01 Track 2, paragraph on group-wise affine quantisation).  The
tests pin the gather against hand values, the single rounding to fp16
against exact rational arithmetic, the rows against the linear oracle with
unit activations, and the round trip against the unquantised table.
"""

from fractions import Fraction

import numpy as np

from oracle import embed as E
from oracle import linear as L
from oracle import rtn as R


def test_hand_values():
    # row 0: group 0 s = 0.5, z = 3; group 1 s = 2, z = 0.25
    q = np.zeros((2, 256), dtype=np.uint8)
    q[0, :4] = [0, 1, 3, 255]
    q[0, 128:130] = [0, 7]
    s = np.array([[0.5, 2.0], [1.0, 1.0]], dtype=np.float16)
    z = np.array([[3.0, 0.25], [0.0, 0.0]], dtype=np.float16)
    out = E.embed(q, s, z, [0, 1, 0], np.float32)
    assert out.shape == (3, 256)
    assert out[0, :4].tolist() == [-1.5, -1.0, 0.0, 126.0]
    assert out[0, 4:128].tolist() == [-1.5] * 124
    assert out[0, 128:130].tolist() == [-0.5, 13.5]
    assert out[0, 130:].tolist() == [-0.5] * 126
    assert np.all(out[1] == 0.0)
    assert np.array_equal(out[2], out[0])


def _exact_fp16(x: Fraction) -> np.float16:
    """The fp16 nearest to the exact rational x (ties to an even significand)."""
    c = np.float16(float(x))
    lo = c if Fraction(float(c)) <= x else np.nextafter(c, np.float16(-np.inf))
    hi = np.nextafter(lo, np.float16(np.inf))
    assert Fraction(float(lo)) <= x <= Fraction(float(hi))
    dl, dh = x - Fraction(float(lo)), Fraction(float(hi)) - x
    if dl != dh:
        return lo if dl < dh else hi
    return lo if (lo.view(np.uint16) & 1) == 0 else hi


def test_single_rounding_to_fp16():
    # values with more significant bits than fp32 holds (small zero points):
    # rounding first to fp32 and then to fp16 can differ from one rounding
    rng = np.random.default_rng(7)
    n = 200000
    q = rng.integers(0, 256, n)
    s = (rng.uniform(0.5, 1.0, n) * 2.0 ** rng.integers(-12, 4, n)).astype(np.float16)
    z = (rng.uniform(0.5, 1.0, n) * 2.0 ** rng.integers(-24, 8, n)).astype(np.float16)
    v = (q - z.astype(np.float64)) * s.astype(np.float64)
    single = v.astype(np.float16)
    double = v.astype(np.float32).astype(np.float16)
    traps = np.nonzero(single != double)[0]
    assert len(traps) > 0, "no double-rounding case in the sample"
    check = np.concatenate([traps, np.arange(2000)])
    for i in check:
        exact = (Fraction(int(q[i])) - Fraction(float(z[i]))) * Fraction(float(s[i]))
        assert Fraction(float(v[i])) == exact            # the fp64 value is exact
        want = _exact_fp16(exact)
        got = E.embed(np.array([[q[i]] * 128], np.uint8), np.array([[s[i]]]), np.array([[z[i]]]), [0])[0, 0]
        assert got.view(np.uint16) == want.view(np.uint16), (i, float(exact))


def test_rows_match_linear_with_unit_activations():
    # y = W x with x = e_k is column k of the dequantised W: the gathered row
    # r is column r of the layer's response to the identity
    rng = np.random.default_rng(3)
    for bits in (3, 4, 6, 8):
        n, k = 9, 256
        q = rng.integers(0, 1 << bits, (n, k)).astype(np.uint8)
        s = rng.uniform(0.001, 0.1, (n, k // 128)).astype(np.float16)
        z = rng.uniform(0, (1 << bits) - 1, (n, k // 128)).astype(np.float16)
        ids = [4, 0, 8, 4]
        got = E.embed(q, s, z, ids, np.float64)
        y = L.linear(q, s, z, np.eye(k))             # [k][n]
        assert np.array_equal(got, y[:, ids].T)


def test_ids_outside_the_table_give_zero_rows():
    q = np.full((3, 128), 200, dtype=np.uint8)
    s = np.full((3, 1), 0.25, dtype=np.float16)
    z = np.full((3, 1), 1.0, dtype=np.float16)
    out = E.embed(q, s, z, [-1, 3, 2, (1 << 31) - 1, 0], np.float16)
    assert np.all(out[[0, 1, 3]] == 0)
    assert np.all(out[[2, 4]] == np.float16(49.75))


def test_round_trip_within_the_rtn_step():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((40, 512)).astype(np.float32) * np.float32(0.02)
    w[:, 17] *= 20.0
    q, s, z = R.rtn(w, 8)
    ids = np.arange(40)[::-1]
    got = E.embed(q, s, z, ids, np.float64)
    step = np.repeat(s.astype(np.float64), 128, axis=1)[ids]
    # half a code step, plus the clamp at the top when s rounded down to fp16
    assert np.all(np.abs(got - w[ids]) <= step * (0.5 + 255 / 1024))
