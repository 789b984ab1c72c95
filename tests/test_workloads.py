"""The seeded input generator: determinism, shapes and the stated recipe."""

import hashlib

import numpy as np

import workloads as W


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    wl = W.WORKLOADS["single_int4"]
    a = W.linear_inputs(0, wl.wid, 0, wl.linears[0], 1)
    b = W.linear_inputs(0, wl.wid, 0, wl.linears[0], 1)
    assert _digest(*a) == _digest(*b)
    c = W.linear_inputs(1, wl.wid, 0, wl.linears[0], 1)
    assert _digest(*a) != _digest(*c)


def test_shapes_and_dtypes():
    wl = W.WORKLOADS["prefill_and_mixed"]
    lin = wl.linears[-1]
    w, x, s, sel = W.linear_inputs(0, wl.wid, len(wl.linears) - 1, lin, 1)
    assert w.shape == (2560, 9728) and w.dtype == np.float32
    assert x.shape == (1, 9728) and x.dtype == np.float16
    assert s.shape == (9728 // 32,) and s.dtype == np.uint32
    assert sel.shape == (40,) and set(sel.tolist()) <= {6, 8} and int((sel == 8).sum()) == 8


def test_outlier_channels():
    rng = W.rng_for(0, 9, 0)
    w = W.weight(1024, 256, rng)
    col_rms = np.sqrt((w.astype(np.float64) ** 2).mean(axis=0))
    big = np.nonzero(col_rms > 0.1)[0]
    assert len(big) == round(0.01 * 1024)
    assert 0.015 < np.median(col_rms) < 0.025


def test_row_sample_matches_full_draw():
    wl = W.WORKLOADS["block_int4"]
    lin = wl.linears[1]  # k_proj 2560 -> 1024
    full = W.linear_inputs(0, wl.wid, 1, lin, 1)[0]
    rows = np.array([0, 5, 511, 1023])
    assert np.array_equal(W.weight_rows(0, wl.wid, 1, lin, rows), full[rows])


def test_sign_bits_are_fair():
    s = W.sign_bits(9728 * 32, W.rng_for(0, 0, 99))
    ones = sum(bin(int(v)).count("1") for v in s)
    n = 9728 * 32
    assert abs(ones - n / 2) < 5 * np.sqrt(n / 4)


def test_trained_scale_zero_stay_valid():
    rng = np.random.default_rng(0)
    s = np.full((4, 3), 0.1, np.float16)
    z = np.full((4, 3), 7, np.float16)
    s2, z2 = W.trained_scale_zero(s, z, rng, 15)
    assert np.all(s2 > 0) and np.all((z2 >= 0) & (z2 <= 15))
    assert np.any(z2.astype(np.float32) != np.round(z2.astype(np.float32)))


def test_scaled_activations_recipe():
    rng = W.rng_for(0, 9, 3)
    x = W.scaled_activations(3, 4096, rng, [1e-3, 1.0, 300.0])
    assert x.dtype == np.float16 and x.shape == (3, 4096)
    rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=1))
    assert np.allclose(rms, [1e-3, 1.0, 300.0], rtol=0.05)
    y = W.scaled_activations(1, 4096, W.rng_for(0, 9, 4), 1.0, outlier_frac=0.01, outlier_scale=50.0)
    big = np.abs(y[0].astype(np.float64)) > 12.0   # beyond any plain N(0, 1) draw of this size
    assert 20 <= int(big.sum()) <= 41
