"""Pins for the oracle's weight rotation and round-to-nearest quantiser.

The model cards fix the affine group form w = (q - z) * s with fp16 scale
and zero per 128 along K (24B0978 Week 01 Track 2, "How these techniques
accelerate inference on CUDA"), round-to-nearest quantisation with group
128 (24B0978 Week 02 Track 2, "Recipe" and "Recipe (exact)"), and that the
rotation folded into the weight leaves the layer's function unchanged
(Week 01 card, paragraph on the random Hadamard transform).  The tests pin
the quantiser by exact rational brute force, closed-form bounds and hand
cases, and the rotation by the invariance of the layer.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import hadamard as H
from oracle import rtn as R

GOLD = os.path.join(os.path.dirname(__file__), "golden", "rtn_cases.json")
BITS = [3, 4, 6, 8]


def _rand_bits(rng, k):
    return rng.integers(0, 1 << 32, size=k // 32, dtype=np.uint64).astype(np.uint32)


def _weights(rng, n, k):
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[:, rng.choice(k, max(1, k // 100), replace=False)] *= 20
    return w


@pytest.mark.parametrize("bits", BITS)
def test_ranges(bits):
    rng = np.random.default_rng(bits)
    q, s, z = R.rtn(_weights(rng, 16, 512), bits)
    qmax = (1 << bits) - 1
    assert q.dtype == np.uint8 and q.max() <= qmax
    assert s.dtype == np.float16 and z.dtype == np.float16
    assert np.all(s.astype(np.float64) > 0)
    zf = z.astype(np.float64)
    assert np.all(zf == np.round(zf)) and zf.min() >= 0 and zf.max() <= qmax


@pytest.mark.parametrize("bits", BITS)
def test_round_trip_within_half_step(bits):
    rng = np.random.default_rng(10 + bits)
    w = _weights(rng, 32, 1024)
    q, s, z = R.rtn(w, bits)
    qmax = (1 << bits) - 1
    g = np.arange(1024) // 128
    sf = s.astype(np.float64)[:, g]
    zf = z.astype(np.float64)[:, g]
    err = np.abs(w.astype(np.float64) - (q.astype(np.float64) - zf) * sf)
    unclamped = (q > 0) & (q < qmax)
    assert np.all(err[unclamped] <= sf[unclamped] / 2 * (1 + 1e-12))
    # clamped codes only happen at the ends of the range, within one step
    assert np.all(err <= sf * (1 + 1e-12))


def _fp16_neighbours(x16):
    a = np.float16(x16)
    return [np.nextafter(a, np.float16(-np.inf)), np.nextafter(a, np.float16(np.inf))]


@pytest.mark.parametrize("bits", BITS)
def test_brute_force_exact(bits):
    """Every code is the nearest grid point, every scale the nearest fp16, in exact arithmetic."""
    rng = np.random.default_rng(20 + bits)
    w = _weights(rng, 3, 256)
    w[0, :128] = np.abs(w[0, :128])          # an all-positive group (lo clamps to 0)
    q, s, z = R.rtn(w, bits)
    qmax = (1 << bits) - 1
    for n in range(w.shape[0]):
        for g in range(2):
            v = [Fraction(float(t)) for t in w[n, 128 * g:128 * (g + 1)]]
            lo, hi = min(min(v), Fraction(0)), max(max(v), Fraction(0))
            target = (hi - lo) / qmax
            sv = Fraction(float(s[n, g]))
            for nb in _fp16_neighbours(s[n, g]):
                assert abs(sv - target) <= abs(Fraction(float(nb)) - target)
            # zero point: nearest integer to -lo/s (ties even), clamped
            zt = -lo / sv
            zc = [c for c in range(qmax + 1)]
            dz = [abs(Fraction(c) - zt) for c in zc]
            best = [c for c in zc if dz[c] == min(dz)]
            want_z = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
            assert float(z[n, g]) == want_z
            zv = Fraction(want_z)
            for i, vi in enumerate(v):
                dist = [abs(vi - (c - zv) * sv) for c in range(qmax + 1)]
                m = min(dist)
                cands = [c for c in range(qmax + 1) if dist[c] == m]
                want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
                assert int(q[n, 128 * g + i]) == want, (n, g, i)


def _group_from_case(c):
    v = np.zeros(128, dtype=np.float32)
    if "linspace" in c:
        return np.linspace(c["linspace"][0], c["linspace"][1], 128).astype(np.float32)
    if c.get("repeat"):
        parts = [np.full(r, h, dtype=np.float32) for h, r in zip(c["head"], c["repeat"])]
        return np.concatenate(parts)
    v[:] = np.float32(c["fill"])
    v[:len(c["head"])] = np.array(c["head"], dtype=np.float32)
    return v


def test_hand_cases():
    cases = json.load(open(GOLD))["cases"]
    for c in cases:
        v = _group_from_case(c)
        q, s, z = R.rtn(v[None, :], c["bits"])
        assert float(s[0, 0]) == c["s"], c["why"]
        assert float(z[0, 0]) == c["z"], c["why"]
        if "q_at" in c:
            for i, want in c["q_at"].items():
                assert int(q[0, int(i)]) == want, c["why"]
        else:
            nh = len(c["head"]) if not c.get("repeat") else 0
            if c.get("repeat"):
                pos = np.cumsum([0] + c["repeat"][:-1])
                for p, want in zip(pos, c["q_head"]):
                    assert int(q[0, p]) == want, c["why"]
            else:
                assert [int(t) for t in q[0, :nh]] == c["q_head"], c["why"]
                assert np.all(q[0, nh:] == c["q_fill"]), c["why"]


def test_per_row_widths():
    rng = np.random.default_rng(30)
    w = _weights(rng, 128, 256)
    rows = np.array([6] * 64 + [8] * 64)
    q, s, z = R.rtn(w, rows)
    q6, s6, z6 = R.rtn(w[:64], 6)
    q8, s8, z8 = R.rtn(w[64:], 8)
    assert np.array_equal(q[:64], q6) and np.array_equal(q[64:], q8)
    assert np.array_equal(s[:64], s6) and np.array_equal(s[64:], s8)
    assert np.array_equal(z[:64], z6) and np.array_equal(z[64:], z8)


def test_rotation_preserves_the_layer():
    rng = np.random.default_rng(31)
    k, n = 1024, 24
    bits = _rand_bits(rng, k)
    w = _weights(rng, n, k)
    x = rng.standard_normal((3, k))
    wp = R.rotate_weight(w, bits, keep_fp64=True)
    lhs = H.rht(x, bits) @ wp.T
    rhs = x @ w.astype(np.float64).T
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12 * np.abs(rhs).max())
    # the rounded weight is the fp32 rounding of that fp64 value
    assert np.array_equal(R.rotate_weight(w, bits), wp.astype(np.float32))


def test_rotation_spreads_outlier_channels():
    # The purpose stated for the rotation: outlier channels get spread over
    # the group, which lowers the quantisation error at a fixed width.
    rng = np.random.default_rng(32)
    k, n = 1024, 64
    bits = _rand_bits(rng, k)
    w = _weights(rng, n, k)
    x = rng.standard_normal((1, k))
    from oracle import linear as L
    y_true = x @ w.astype(np.float64).T
    q0, s0, z0 = R.rtn(w, 4)
    e_plain = np.linalg.norm(L.linear(q0, s0, z0, x) - y_true)
    q1, s1, z1 = R.prepare(w, bits, 4)
    e_rot = np.linalg.norm(L.linear(q1, s1, z1, x, bits) - y_true)
    assert e_rot < 0.8 * e_plain
